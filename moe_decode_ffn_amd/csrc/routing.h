// routing.h -- top-k ranking of one token by one wave, and bucketing of the
// (token, slot) pairs by expert inside one workgroup (the router launch's
// routing tail).
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

// LDS words one wave needs for ranking: key, index, value of up to kMaxTopK
// picks (16-byte aligned).
constexpr int kRankWords = 3 * 32;

// One wave ranks one token.  lg: E+1 logits (column E = shared-gate logit);
// wlds: kRankWords words of 16-byte-aligned LDS owned by this wave.
//   1. radix select: the k-th largest key P, two bits at a time from the top,
//      counting keys >= candidate with one ballot per element slot;
//   2. selected = keys above P, plus the lowest-index keys equal to P until k;
//   3. the k picks are compacted into LDS and lane j < k ranks pick j against
//      the others (key descending, index ascending) -> its slot.
// Weights: p_e = exp(l_e - max l) / sum_all exp(.) renormalised over the picks
// is w_j = exp(l_j - m) / sum_picks exp(l_i - m) for any m (the full sum
// cancels); m = the largest pick, which is also the largest logit.
template <int EPL>
__device__ void route_token(const float *lg, int E, int k, int lane, uint32_t *wlds, const RouteOut &o) {
    float v[EPL];
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        v[i] = e < E ? lg[e] : -INFINITY;
        key[i] = e < E ? logit_key(v[i]) : 0u;  // padding sorts below every logit
    }
    const float glog = lg[E];

    // 1. k-th largest key, two bits per round (three independent counts)
    uint32_t P = 0;
    for (int b = 30; b >= 0; b -= 2) {
        const uint32_t c1 = P | (1u << b), c2 = P | (2u << b), c3 = P | (3u << b);
        int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            n1 += __popcll(__ballot(key[i] >= c1));
            n2 += __popcll(__ballot(key[i] >= c2));
            n3 += __popcll(__ballot(key[i] >= c3));
        }
        P = n3 >= k ? c3 : n2 >= k ? c2 : n1 >= k ? c1 : P;
    }
    // 2. selection: everything above P, then ties at P in index order
    int above = 0;
    unsigned long long eqm[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        above += __popcll(__ballot(key[i] > P));
        eqm[i] = __ballot(key[i] == P);
    }
    const int need = k - above;  // >= 1
    const unsigned long long below = (1ull << lane) - 1ull;
    int eq_before = 0;  // ties at P with a lower index than this lane's first slot
#pragma unroll
    for (int i = 0; i < EPL; ++i) eq_before += __popcll(eqm[i] & below);
    bool sel[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const bool eq = key[i] == P;
        sel[i] = key[i] > P || (eq && eq_before < need);
        eq_before += eq ? 1 : 0;
    }
    // 3. compaction in index order, then rank among the picks
    int pos = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) pos += __popcll(__ballot(sel[i]) & below);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if (sel[i]) {
            wlds[pos] = key[i];
            wlds[32 + pos] = (uint32_t)(lane * EPL + i);
            wlds[64 + pos] = __float_as_uint(v[i]);
            ++pos;
        }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float myp = 0.f;
    int myid = 0, slot = 0;
    if (lane < k) {
        const uint32_t mk = wlds[lane], mi = wlds[32 + lane];
        const uint4 *k4 = reinterpret_cast<const uint4 *>(wlds);
        const uint4 *i4 = reinterpret_cast<const uint4 *>(wlds + 32);
        const uint4 *v4 = reinterpret_cast<const uint4 *>(wlds + 64);
        float m = -INFINITY;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (4 * q < k) {
                const uint4 kk = k4[q], ii = i4[q], vv = v4[q];
                const uint32_t ka[4] = {kk.x, kk.y, kk.z, kk.w}, ia[4] = {ii.x, ii.y, ii.z, ii.w};
                const uint32_t va[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * q + r < k) {
                        slot += (ka[r] > mk || (ka[r] == mk && ia[r] < mi)) ? 1 : 0;
                        m = fmaxf(m, __uint_as_float(va[r]));
                    }
            }
        }
        myid = (int)mi;
        myp = expf(__uint_as_float(wlds[64 + lane]) - m);
    }
    const float psum = seg_sum<64>(lane < k ? myp : 0.f);
    if (lane < k) {
        const float w = myp / psum;
        o.ids[slot] = myid;
        o.w[slot] = w;
        if (o.dbg_ids) o.dbg_ids[slot] = myid;
        if (o.dbg_w) o.dbg_w[slot] = w;
    }
    if (lane == 0) {
        const float s = sigmoid_f(glog);
        o.gate[0] = s;
        if (o.dbg_gate) o.dbg_gate[0] = s;
    }
    if (o.dbg_logits)
        for (int e = lane; e < E; e += 64) o.dbg_logits[e] = lg[e];
    // the wave's LDS is reused by its next token
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void route_token_any(const float *lg, int E, int k, int lane, uint32_t *wlds,
                                                const RouteOut &o) {
    const int epl = (E + 63) / 64;
    if (epl <= 1) route_token<1>(lg, E, k, lane, wlds, o);
    else if (epl <= 2) route_token<2>(lg, E, k, lane, wlds, o);
    else if (epl <= 4) route_token<4>(lg, E, k, lane, wlds, o);
    else route_token<8>(lg, E, k, lane, wlds, o);
}

// LDS ints the bucketing needs for E experts and T tokens.
__host__ __device__ inline int bucket_scratch_ints(int E, int T) {
    return E * ((T + 31) / 32) + 2 * E + 2 * 16 + 16;
}

// Bucketing of up to 64 pairs by one wave (same results as bucket_pairs):
// lane q holds pair q; its position is the number of pairs with a smaller
// expert plus the pairs of the same expert with a smaller pair id.
__device__ inline void bucket_pairs_wave(const int *ids, int NP, int E, int4 *slots, int *pairs,
                                         int *pos_expert, int *n_unique) {
    const int lane = threadIdx.x & 63;
    const int e = lane < NP ? ids[lane] : 0x7fffffff;
    const bool ok = lane < NP && e >= 0 && e < E;
    // ids is 16-byte aligned and the LDS behind it is readable, so it is read
    // four entries at a time; entries at or past NP are masked out
    const int4 *ids4 = reinterpret_cast<const int4 *>(ids);
    int smaller = 0, same_before = 0, same = 0;
#pragma unroll 4
    for (int j0 = 0; j0 < NP; j0 += 4) {
        const int4 q = ids4[j0 >> 2];
        const int qa[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + r, ej = qa[r];
            const bool vj = j < NP && ej >= 0 && ej < E;  // an out-of-range id takes no position
            smaller += (vj && ej < e) ? 1 : 0;
            same += (vj && ej == e) ? 1 : 0;
            same_before += (vj && ej == e && j < lane) ? 1 : 0;
        }
    }
    const bool first = ok && same_before == 0;
    const unsigned long long fm = __ballot(first);
    // slot of this lane's expert: first lanes of smaller experts
    int u = 0;
#pragma unroll 4
    for (int j0 = 0; j0 < NP; j0 += 4) {
        const int4 q = ids4[j0 >> 2];
        const int qa[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + r;
            u += (j < NP && ((fm >> j) & 1ull) && qa[r] < e) ? 1 : 0;
        }
    }
    if (ok) {
        pairs[smaller + same_before] = lane;
        pos_expert[smaller + same_before] = e;
    }
    if (first) slots[u] = make_int4(e, smaller, same, 0);
    if (lane == 0) *n_unique = __popcll(fm);
}

// Bucketing of all T*k pairs by one workgroup (any multiple of 64 threads up
// to 1024).  ids[] may be in LDS or global memory.  Outputs (any memory):
// slots[u] = (expert, first position, count, 0) for used experts in ascending
// order, pairs[pos] = t*k + j, pos_expert[pos], *n_unique.  Positions are
// expert-major, tokens ascending within an expert; a token's rank in its
// expert's bucket is the number of earlier tokens in the expert's token bitmap
// (a token picks an expert at most once).  Integer only: the result is unique.
__device__ void bucket_pairs(const int *ids, int T, int k, int E, uint32_t *scratch, int4 *slots,
                             int *pairs, int *pos_expert, int *n_unique) {
    const int nth = blockDim.x, nw = nth >> 6;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NP = T * k, W = (T + 31) / 32;
    uint32_t *mask = scratch;                     // [E][W] token bitmaps
    int *cnt = (int *)(mask + (size_t)E * W);     // [E]
    int *off = cnt + E;                           // [E] first position of expert e
    int *wtot = off + E;                          // [2 * 16] wave totals
    for (int i = tid; i < E * W; i += nth) mask[i] = 0u;
    __syncthreads();
    for (int q = tid; q < NP; q += nth) {
        const int t = q / k, e = ids[q];
        if (e >= 0 && e < E) atomicOr(&mask[e * W + (t >> 5)], 1u << (t & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += nth) {
        int c = 0;
        for (int w = 0; w < W; ++w) c += __popc(mask[e * W + w]);
        cnt[e] = c;
    }
    __syncthreads();
    // exclusive scans of cnt[] and (cnt[] > 0); thread owns EPT consecutive experts
    const int EPT = (E + nth - 1) / nth;
    int a = 0, b = 0;
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < E) { a += cnt[e]; b += cnt[e] > 0; }
    }
    int ia = a, ib = b;
    for (int d = 1; d < 64; d <<= 1) {
        const int ya = __shfl_up(ia, d), yb = __shfl_up(ib, d);
        if (lane >= d) { ia += ya; ib += yb; }
    }
    if (lane == 63) { wtot[wave] = ia; wtot[16 + wave] = ib; }
    __syncthreads();
    int ba = ia - a, bb = ib - b;
    for (int w = 0; w < wave; ++w) { ba += wtot[w]; bb += wtot[16 + w]; }
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < E) {
            off[e] = ba;
            if (cnt[e] > 0) slots[bb] = make_int4(e, ba, cnt[e], 0);
            ba += cnt[e];
            bb += cnt[e] > 0;
        }
    }
    if (tid == nth - 1) {
        int nu = 0;
        for (int w = 0; w < nw; ++w) nu += wtot[16 + w];
        *n_unique = nu;
    }
    __syncthreads();
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
// local tables the job records, weights and gates also live in LDS (a
// workgroup that routes for its own use); without, they only go to memory.
struct RouteLds {
    size_t ids, pairs, pose, nu, slots, records, scratch, rank, w, g, bytes;
    bool local;
};

__host__ __device__ inline RouteLds route_lds_layout(int T, int k, int E, int waves, bool local) {
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
    L.scratch = o; o += (size_t)bucket_scratch_ints(E, T) * 4;
    o = (o + 15) & ~(size_t)15;
    L.rank = o;    o += (size_t)waves * kRankWords * 4;
    if (local) {
        L.records = o; o += ns * kRecInts * 4;
        L.w = o;       o += np * 4;
        L.g = o;       o += (size_t)T * 4;
    }
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
// gates go to g when g.wts is set, else to LDS.  No barrier inside.
__device__ inline void rank_tokens(const float *logits, int t_lo, int t_hi, int E, int k, uint8_t *area,
                                   const RouteLds &L, const RouteGlobal &g, bool ids_to_global) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int *ids = reinterpret_cast<int *>(area + L.ids);
    float *lw = reinterpret_cast<float *>(area + L.w);
    float *lg = reinterpret_cast<float *>(area + L.g);
    uint32_t *rank = reinterpret_cast<uint32_t *>(area + L.rank) + wave * kRankWords;
    for (int t = t_lo + wave; t < t_hi; t += nw) {
        RouteOut o{(ids_to_global ? g.ids : ids) + t * k, (g.wts ? g.wts : lw) + t * k,
                   (g.gate_s ? g.gate_s : lg) + t,
                   g.dbg_ids ? g.dbg_ids + t * k : nullptr, g.dbg_w ? g.dbg_w + t * k : nullptr,
                   g.dbg_gate ? g.dbg_gate + t : nullptr,
                   g.dbg_logits ? g.dbg_logits + (size_t)t * E : nullptr};
        route_token_any(logits + (size_t)t * (E + 1), E, k, lane, rank, o);
    }
}

// With every id in LDS: buckets the pairs and builds the job records in LDS;
// copies the tables to g where its pointers are set.  Barriers inside: call
// from every thread of the workgroup.  Returns the used-expert count.
__device__ inline int bucket_tokens(int T, int k, int E, uint8_t *area, const RouteLds &L,
                                    const RouteGlobal &g) {
    const int tid = threadIdx.x, NP = T * k;
    int *ids = reinterpret_cast<int *>(area + L.ids);
    int *pairs = reinterpret_cast<int *>(area + L.pairs);
    int *pose = reinterpret_cast<int *>(area + L.pose);
    int *nup = reinterpret_cast<int *>(area + L.nu);
    int4 *slots = reinterpret_cast<int4 *>(area + L.slots);
    int *rec = reinterpret_cast<int *>(area + L.records);
    __syncthreads();
    if (NP <= 16) {  // measured: one wave wins up to 16 pairs, the whole workgroup above
        if (threadIdx.x < 64) bucket_pairs_wave(ids, NP, E, slots, pairs, pose, nup);
    } else {
        bucket_pairs(ids, T, k, E, reinterpret_cast<uint32_t *>(area + L.scratch), slots, pairs, pose, nup);
    }
    __syncthreads();
    const int nu = *nup;
    for (int i = tid; i < nu * kRecInts; i += blockDim.x) {
        const int u = i / kRecInts, f = i - u * kRecInts;
        const int4 sv = slots[u];
        int v;
        if (f == 0) v = sv.x;
        else if (f == 1) v = sv.y;
        else if (f == 2) v = sv.z;
        else if (f == 3) v = 0;
        else v = (f - 4 < sv.z) ? pairs[sv.y + f - 4] : -1;
        if (L.local) rec[i] = v;
        if (g.records) g.records[i] = v;
    }
    if (g.ids)
        for (int i = tid; i < NP; i += blockDim.x) {
            g.ids[i] = ids[i];
            g.pairs[i] = pairs[i];
            g.pos_expert[i] = pose[i];
        }
    if (g.n_unique && tid == 0) *g.n_unique = nu;
    __syncthreads();
    return nu;
}

}  // namespace moeffn

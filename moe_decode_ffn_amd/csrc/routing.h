// routing.h -- top-k ranking of one token by one wave, and bucketing of the
// (token, slot) pairs by expert inside one workgroup.  Used by the router's
// ticket path (larger batches) and by the routed gate/up workgroups, which
// rank the batch themselves in the small-batch regime.
//
// Ranking: experts ordered by (logit descending, index ascending); ids are the
// first k in that order; p = softmax over all experts; w_j = p_j / sum_j p_j.
// The pages print no routing formula; this is the plain reading of "softmax,
// top-k, renormalise" with exact ties going to the lower expert index.
#pragma once

#include "device.h"

namespace moeffn {

struct RouteOut {
    int *ids;        // [k]
    float *w;        // [k]
    float *gate;     // [1] sigmoid(logit of the gate vector)
    int32_t *dbg_ids;
    float *dbg_w, *dbg_gate, *dbg_logits;
};

// One wave ranks one token.  lg: E+1 logits (column E = shared-gate logit).
template <int EPL>
__device__ void route_token(const float *lg, int E, int k, int lane, const RouteOut &o) {
    // blocked layout: lane l holds experts l*EPL .. l*EPL+EPL-1, so a lower
    // lane always holds lower indices
    float v[EPL];
    int ix[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        v[i] = e < E ? lg[e] : -INFINITY;
        ix[i] = e < E ? e : 0x7fffffff;
    }
    const float glog = lg[E];
    float lm = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) lm = fmaxf(lm, v[i]);
    const float m = wave_max(lm);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if (ix[i] < E) z += expf(v[i] - m);
    z = seg_sum<64>(z);
    // local order: (value desc, index asc)
#pragma unroll
    for (int pass = 0; pass < EPL; ++pass) {
#pragma unroll
        for (int b = 0; b + 1 < EPL; ++b) {
            const bool better = v[b + 1] > v[b] || (v[b + 1] == v[b] && ix[b + 1] < ix[b]);
            if (better) {
                const float tv = v[b]; v[b] = v[b + 1]; v[b + 1] = tv;
                const int ti = ix[b]; ix[b] = ix[b + 1]; ix[b + 1] = ti;
            }
        }
    }
    float myp = 0.f;
    int myid = 0;
    for (int j = 0; j < k; ++j) {
        const bool has = ix[0] < E;
        const float head = has ? v[0] : -INFINITY;
        const float hm = wave_max(head);
        unsigned long long mask = __ballot(has && head == hm);
        if (mask == 0ull) mask = __ballot(has);  // only if logits are NaN
        const int wl = __ffsll(mask) - 1;
        const int id = __shfl(ix[0], wl);
        const float hv = __shfl(v[0], wl);
        if (lane == wl) {
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) { v[i] = v[i + 1]; ix[i] = ix[i + 1]; }
            v[EPL - 1] = -INFINITY;
            ix[EPL - 1] = 0x7fffffff;
        }
        const float pj = expf(hv - m) / z;  // softmax probability of the j-th pick
        if (lane == j) { myp = pj; myid = id; }
    }
    const float psum = seg_sum<64>(lane < k ? myp : 0.f);
    if (lane < k) {
        const float w = myp / psum;
        o.ids[lane] = myid;
        o.w[lane] = w;
        if (o.dbg_ids) o.dbg_ids[lane] = myid;
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

__device__ __forceinline__ void route_token_any(const float *lg, int E, int k, int lane,
                                                const RouteOut &o) {
    const int epl = (E + 63) / 64;
    if (epl <= 1) route_token<1>(lg, E, k, lane, o);
    else if (epl <= 2) route_token<2>(lg, E, k, lane, o);
    else if (epl <= 4) route_token<4>(lg, E, k, lane, o);
    else route_token<8>(lg, E, k, lane, o);
}

// LDS ints the bucketing needs for E experts and T tokens.
__host__ __device__ inline int bucket_scratch_ints(int E, int T) {
    return E * ((T + 31) / 32) + 2 * E + 2 * 16 + 16;
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

}  // namespace moeffn

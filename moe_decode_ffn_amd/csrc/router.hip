// router.hip -- router GEMV, softmax, top-k, renormalisation and
// token-to-expert bucketing in one launch.
//
// Grid (row tiles x token tiles).  Every workgroup computes the logits of its
// router rows for its token tile (row E is the shared-expert gate vector, so
// its logit is sigma's argument).  The last workgroup to finish a token tile
// (integer ticket, no spinning) ranks that tile's tokens, one wave per token;
// the last tile to finish then buckets all (token, slot) pairs by expert.
// Tickets reset themselves, so a forward leaves the counters at zero and the
// launch can be captured and replayed.
//
// Ranking: experts ordered by (logit descending, index ascending); the pages
// print no routing formula, the reading taken is softmax over all experts,
// keep the k largest, renormalise over them (weights w_j = p_j / sum p).
#include "device.h"
#include "internal.h"

namespace moeffn {

constexpr int kRouterWaves = 4;

int router_rows_per_wg(const RowMap &m) { return kRouterWaves * (64 / m.lpr); }

// ---- ranking of one token by one wave -------------------------------------------
template <int EPL>
__device__ void route_token(const RouterParams &p, int t, int lane) {
    const int E = p.E, k = p.k;
    const float *lg = p.logits + (size_t)t * (E + 1);
    // blocked layout: lane l holds experts l*EPL .. l*EPL+EPL-1, so a lower lane
    // always holds lower indices
    float v[EPL];
    int ix[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        v[i] = e < E ? lg[e] : -INFINITY;
        ix[i] = e < E ? e : 0x7fffffff;
    }
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
        p.ids[t * k + lane] = myid;
        p.wts[t * k + lane] = w;
        if (p.dbg_ids) p.dbg_ids[t * k + lane] = myid;
        if (p.dbg_w) p.dbg_w[t * k + lane] = w;
    }
    if (lane == 0) {
        const float s = sigmoid_f(lg[E]);
        p.gate_s[t] = s;
        if (p.dbg_gate) p.dbg_gate[t] = s;
    }
    if (p.dbg_logits)
        for (int e = lane; e < E; e += 64) p.dbg_logits[(size_t)t * E + e] = lg[e];
}

__device__ void route_token_any(const RouterParams &p, int t, int lane) {
    const int epl = (p.E + 63) / 64;
    if (epl <= 1) route_token<1>(p, t, lane);
    else if (epl <= 2) route_token<2>(p, t, lane);
    else if (epl <= 4) route_token<4>(p, t, lane);
    else route_token<8>(p, t, lane);
}

// ---- bucketing of all pairs by the whole workgroup -------------------------------------
// Positions: expert-major (experts ascending), tokens ascending inside an
// expert.  A token appears at most once per expert (top-k picks distinct
// experts), so its rank inside the bucket is the number of earlier tokens in
// the expert's token bitmap.
__device__ void bucket_pairs(const RouterParams &p, uint32_t *lds) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = p.E, T = p.T, k = p.k, NP = T * k, W = (T + 31) / 32;
    uint32_t *mask = lds;                       // [E][W] token bitmaps
    int *cnt = (int *)(mask + (size_t)E * W);   // [E]
    int *off = cnt + E;                         // [E] first position of expert e
    int *uoff = off + E;                        // [E] slot of expert e among used experts
    int *wtot = uoff + E;                       // [2 * waves]
    for (int i = tid; i < E * W; i += 256) mask[i] = 0u;
    __syncthreads();
    for (int q = tid; q < NP; q += 256) {
        const int t = q / k, e = p.ids[q];
        if (e >= 0 && e < E) atomicOr(&mask[e * W + (t >> 5)], 1u << (t & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
        int c = 0;
        for (int w = 0; w < W; ++w) c += __popc(mask[e * W + w]);
        cnt[e] = c;
    }
    __syncthreads();
    // exclusive scans of cnt[] and (cnt[] > 0) over experts; thread owns EPT experts
    const int EPT = (E + 255) / 256;
    int a = 0, b = 0;
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < E) { a += cnt[e]; b += cnt[e] > 0; }
    }
    int ia = a, ib = b;  // inclusive wave scans
    for (int d = 1; d < 64; d <<= 1) {
        const int ya = __shfl_up(ia, d), yb = __shfl_up(ib, d);
        if (lane >= d) { ia += ya; ib += yb; }
    }
    if (lane == 63) { wtot[wave] = ia; wtot[kRouterWaves + wave] = ib; }
    __syncthreads();
    int ba = ia - a, bb = ib - b;  // exclusive within the wave
    for (int w = 0; w < wave; ++w) { ba += wtot[w]; bb += wtot[kRouterWaves + w]; }
    for (int i = 0; i < EPT; ++i) {
        const int e = tid * EPT + i;
        if (e < E) {
            off[e] = ba;
            uoff[e] = bb;
            if (cnt[e] > 0) p.slots[bb] = make_int4(e, ba, cnt[e], 0);
            ba += cnt[e];
            bb += cnt[e] > 0;
        }
    }
    if (tid == 255) {
        int nu = 0;
        for (int w = 0; w < kRouterWaves; ++w) nu += wtot[kRouterWaves + w];
        *p.n_unique = nu;
    }
    __syncthreads();
    for (int q = tid; q < NP; q += 256) {
        const int t = q / k, e = p.ids[q];
        if (e < 0 || e >= E) continue;
        const uint32_t *me = mask + e * W;
        int rank = __popc(me[t >> 5] & ((1u << (t & 31)) - 1u));
        for (int w = 0; w < (t >> 5); ++w) rank += __popc(me[w]);
        const int pos = off[e] + rank;
        p.pairs[pos] = q;
        p.pos_expert[pos] = e;
    }
}

// ---- the router kernel --------------------------------------------------------------
template <int LPR, int NC, bool XBF>
__global__ __launch_bounds__(256) void k_router(RouterParams p) {
    constexpr int RPI = 64 / LPR;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, sl = lane % LPR;
    const int H = p.H, E = p.E;
    const int n_chunks = H / 4;  // fp32 rows, 4 elements per 16-byte chunk
    const int row = (blockIdx.x * kRouterWaves + wave) * RPI + seg;
    const bool valid = row <= E;
    const float *W = row < E ? p.router + (size_t)row * H : p.gate_vec;

    float4 w[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = sl + LPR * n;
        w[n] = (valid && c < n_chunks) ? *reinterpret_cast<const float4 *>(W + 4 * c)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int t0 = blockIdx.y * p.tok_tile;
    const int nt = min(p.tok_tile, p.T - t0);
    const int xrow = H * (XBF ? 2 : 4);
    const uint8_t *xs = (const uint8_t *)p.x + (size_t)t0 * xrow;
    for (int i = tid; i < nt * xrow / 16; i += 256)
        reinterpret_cast<uint4 *>(lds)[i] = ld16(xs + 16 * (size_t)i);
    __syncthreads();

    for (int i = 0; i < nt; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const int c = sl + LPR * n;
            if (c < n_chunks) {
                float4 xv;
                if constexpr (XBF) {
                    const uint2 b = *reinterpret_cast<const uint2 *>(lds + i * xrow + 8 * c);
                    xv = make_float4(bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y));
                } else {
                    xv = *reinterpret_cast<const float4 *>(lds + i * xrow + 16 * c);
                }
                acc = fmaf(w[n].x, xv.x, acc);
                acc = fmaf(w[n].y, xv.y, acc);
                acc = fmaf(w[n].z, xv.z, acc);
                acc = fmaf(w[n].w, xv.w, acc);
            }
        }
        acc = seg_sum<LPR>(acc);
        if (valid && sl == 0) p.logits[(size_t)(t0 + i) * (E + 1) + row] = acc;
    }

    // ticket of this token tile: the last row workgroup ranks the tile's tokens
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        s_last = atomicAdd(&p.counters[blockIdx.y], 1) == (int)gridDim.x - 1;
        __threadfence();
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int i = wave; i < nt; i += kRouterWaves) route_token_any(p, t0 + i, lane);
    if (tid == 0) atomicExch(&p.counters[blockIdx.y], 0);

    // ticket over token tiles: the last tile buckets every pair
    __threadfence();
    __syncthreads();
    if (gridDim.y > 1) {
        if (tid == 0) {
            s_last = atomicAdd(&p.counters[gridDim.y], 1) == (int)gridDim.y - 1;
            __threadfence();
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        if (tid == 0) atomicExch(&p.counters[gridDim.y], 0);
    }
    bucket_pairs(p, reinterpret_cast<uint32_t *>(lds));
}

template <int LPR, int NC>
static hipError_t launch_router_t(const RouterParams &p, int grid_rows, int grid_tiles,
                                  hipStream_t s) {
    const size_t stage = (size_t)p.tok_tile * p.H * (p.x_bf16 ? 2 : 4);
    const size_t bucket = (size_t)p.E * ((p.T + 31) / 32 + 3) * 4 + 64;
    const size_t lds = stage > bucket ? stage : bucket;
    const dim3 grid(grid_rows, grid_tiles);
    if (p.x_bf16)
        hipLaunchKernelGGL((k_router<LPR, NC, true>), grid, dim3(256), lds, s, p);
    else
        hipLaunchKernelGGL((k_router<LPR, NC, false>), grid, dim3(256), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_router(const RouterParams &p, const RowMap &m, int grid_rows, int grid_tiles,
                         hipStream_t s) {
    if (grid_tiles + 1 > kCounterInts) return hipErrorInvalidValue;
    switch (m.lpr * 100 + m.nc) {
    case 801: return launch_router_t<8, 1>(p, grid_rows, grid_tiles, s);
    case 1601: return launch_router_t<16, 1>(p, grid_rows, grid_tiles, s);
    case 3201: return launch_router_t<32, 1>(p, grid_rows, grid_tiles, s);
    case 6401: return launch_router_t<64, 1>(p, grid_rows, grid_tiles, s);
    case 6402: return launch_router_t<64, 2>(p, grid_rows, grid_tiles, s);
    case 6404: return launch_router_t<64, 4>(p, grid_rows, grid_tiles, s);
    case 6408: return launch_router_t<64, 8>(p, grid_rows, grid_tiles, s);
    case 6416: return launch_router_t<64, 16>(p, grid_rows, grid_tiles, s);
    case 6432: return launch_router_t<64, 32>(p, grid_rows, grid_tiles, s);
    default: return hipErrorInvalidValue;
    }
}

// ---- bounded delay (test hook) ------------------------------------------------------
__global__ void k_delay(uint64_t ticks) {
    const uint64_t t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

hipError_t launch_delay(hipStream_t s, uint64_t ticks) {
    hipLaunchKernelGGL(k_delay, dim3(1), dim3(64), 0, s, ticks);
    return hipGetLastError();
}

}  // namespace moeffn

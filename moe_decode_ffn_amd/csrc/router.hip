// router.hip -- router GEMV (fp32 rows, row E = the shared-expert gate vector)
// and, for batches above the small-batch limit, ranking and bucketing in the
// same launch.
//
// Small batches: the launch only writes the logits [T][E+1]; the routed
// gate/up workgroups rank the batch themselves (routing.h), one dependent
// memory round trip instead of three.
// Larger batches (ticket path): the last workgroup of each token tile
// (integer ticket, no spinning) ranks that tile's tokens, one wave per token;
// the last tile then buckets every (token, slot) pair.  Each workgroup makes
// its logits visible with one device-scope fence after all its stores have
// completed, and tickets reset themselves, so the launch can be replayed.
#include "device.h"
#include "internal.h"
#include "routing.h"

namespace moeffn {

constexpr int kRouterWaves = 4;

int router_rows_per_wg(const RowMap &m) { return kRouterWaves * (64 / m.lpr); }

template <int LPR, int NC, bool XBF>
__global__ __launch_bounds__(256) void k_router(RouterParams p) {
    constexpr int RPI = 64 / LPR;
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, sl = lane % LPR;
    const int H = p.H, E = p.E, k = p.k;
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
    if (!p.route) return;

    // ---- ticket path ------------------------------------------------------------------
    __builtin_amdgcn_s_waitcnt(0);  // every store of this workgroup has completed
    __syncthreads();
    if (tid == 0) {
        __threadfence();  // one device-scope release for the workgroup
        s_last = atomicAdd(&p.counters[blockIdx.y], 1) == (int)gridDim.x - 1;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    int *r_ids = reinterpret_cast<int *>(lds);  // staging area is free now
    for (int i = wave; i < nt; i += kRouterWaves) {
        const int t = t0 + i;
        RouteOut o{p.ids + t * k, p.wts + t * k, p.gate_s + t,
                   p.dbg_ids ? p.dbg_ids + t * k : nullptr, p.dbg_w ? p.dbg_w + t * k : nullptr,
                   p.dbg_gate ? p.dbg_gate + t : nullptr,
                   p.dbg_logits ? p.dbg_logits + (size_t)t * E : nullptr};
        route_token_any(p.logits + (size_t)t * (E + 1), E, k, lane, o);
    }
    if (tid == 0) atomicExch(&p.counters[blockIdx.y], 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (gridDim.y > 1) {
        if (tid == 0) {
            __threadfence();
            s_last = atomicAdd(&p.counters[gridDim.y], 1) == (int)gridDim.y - 1;
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        if (tid == 0) atomicExch(&p.counters[gridDim.y], 0);
    }
    // all ids of the batch into LDS, then bucket them there
    const int NP = p.T * k;
    for (int q = tid; q < NP; q += 256) r_ids[q] = p.ids[q];
    __syncthreads();
    bucket_pairs(r_ids, p.T, k, E, reinterpret_cast<uint32_t *>(r_ids + NP), p.slots, p.pairs,
                 p.pos_expert, p.n_unique);
}

size_t router_lds_bytes(const RouterParams &p) {
    const size_t stage = (size_t)p.tok_tile * p.H * (p.x_bf16 ? 2 : 4);
    const size_t route = p.route ? (size_t)(p.T * p.k + bucket_scratch_ints(p.E, p.T)) * 4 : 0;
    return stage > route ? stage : route;
}

template <int LPR, int NC>
static hipError_t launch_router_t(const RouterParams &p, int grid_rows, int grid_tiles,
                                  hipStream_t s) {
    const size_t lds = router_lds_bytes(p);
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
    if (router_lds_bytes(p) > kLdsLimit) return hipErrorInvalidValue;
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

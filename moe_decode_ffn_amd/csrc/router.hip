// router.hip -- router GEMV (fp32 rows; row E is the shared-expert gate
// vector, so its logit is sigma's argument) and the routing kernel.
//
// k_router: logits [T][E+1]; workgroups tile (rows x tokens), no cross-
//   workgroup communication.
// k_route: one workgroup of 1024 threads ranks every token (one wave per
//   token, routing.h), buckets the (token, slot) pairs by expert and writes
//   the tables the expert kernels read: ids and weights per slot, the gate
//   value per token, and one 64-byte job record per used expert
//   (expert, first position, count, 0, first 12 pair ids) so an expert
//   workgroup learns everything about its job from one scalar load.
#include "device.h"
#include "internal.h"
#include "routing.h"

namespace moeffn {

constexpr int kRouterWaves = 4;
constexpr int kRouteThreads = 1024;

int router_rows_per_wg(const RowMap &m) { return kRouterWaves * (64 / m.lpr); }

template <int LPR, int NC, bool XBF>
__global__ __launch_bounds__(256) void k_router(RouterParams p) {
    constexpr int RPI = 64 / LPR;
    extern __shared__ __align__(16) uint8_t lds[];
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
}

__global__ __launch_bounds__(kRouteThreads) void k_route(RouteParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int T = p.T, E = p.E, k = p.k, NP = T * k;
    int *r_ids = reinterpret_cast<int *>(lds);       // [NP]
    int *r_pairs = r_ids + NP;                       // [NP]
    int *r_pose = r_pairs + NP;                      // [NP]
    int *r_nu = r_pose + NP;                         // [4]
    int4 *r_slots = reinterpret_cast<int4 *>(lds + (((size_t)(3 * NP + 4) * 4 + 15) & ~(size_t)15));
    uint32_t *scratch = reinterpret_cast<uint32_t *>(r_slots + (E < NP ? E : NP));

    for (int t = wave; t < T; t += nw) {
        RouteOut o{r_ids + t * k, p.wts + t * k, p.gate_s + t,
                   p.dbg_ids ? p.dbg_ids + t * k : nullptr, p.dbg_w ? p.dbg_w + t * k : nullptr,
                   p.dbg_gate ? p.dbg_gate + t : nullptr,
                   p.dbg_logits ? p.dbg_logits + (size_t)t * E : nullptr};
        route_token_any(p.logits + (size_t)t * (E + 1), E, k, lane, o);
    }
    __syncthreads();
    bucket_pairs(r_ids, T, k, E, scratch, r_slots, r_pairs, r_pose, r_nu);
    __syncthreads();
    const int nu = *r_nu;
    for (int i = tid; i < NP; i += blockDim.x) {
        p.ids[i] = r_ids[i];
        p.pairs[i] = r_pairs[i];
        p.pos_expert[i] = r_pose[i];
    }
    for (int i = tid; i < nu * kRecInts; i += blockDim.x) {
        const int u = i / kRecInts, f = i - u * kRecInts;
        const int4 s = r_slots[u];
        int v;
        if (f == 0) v = s.x;
        else if (f == 1) v = s.y;
        else if (f == 2) v = s.z;
        else if (f == 3) v = 0;
        else v = (f - 4 < s.z) ? r_pairs[s.y + f - 4] : -1;
        p.records[i] = v;
    }
    if (tid == 0) *p.n_unique = nu;
}

size_t router_lds_bytes(const RouterParams &p) {
    return (size_t)p.tok_tile * p.H * (p.x_bf16 ? 2 : 4);
}

size_t route_lds_bytes(int T, int k, int E) {
    const int np = T * k;
    return (((size_t)(3 * np + 4) * 4 + 15) & ~(size_t)15) + (size_t)(E < np ? E : np) * 16 +
           (size_t)bucket_scratch_ints(E, T) * 4;
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

hipError_t launch_route(const RouteParams &p, hipStream_t s) {
    const size_t lds = route_lds_bytes(p.T, p.k, p.E);
    if (lds > kLdsLimit) return hipErrorInvalidValue;
    // one wave per token up to 16 waves
    const int waves = p.T < 16 ? (p.T < 4 ? 4 : p.T) : 16;
    hipLaunchKernelGGL(k_route, dim3(1), dim3(64 * waves), lds, s, p);
    return hipGetLastError();
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

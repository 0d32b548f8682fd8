// router.hip -- the router (fp32 rows; row E is the shared-expert gate vector, so
// its logit is sigma's argument) and the routing launches.
//
// Logits: a GEMV over (rows x token tiles) for small batches, bf16 tokens with the
// input norm or fp32 tokens; an MFMA GEMM over an exact bf16 split of the rows above
// 16 bf16 tokens.  Where the routing runs depends on the batch: in every gate/up
// workgroup (a few tokens), in k_route (one wave per token, up to 16 tokens), or in
// the batch launches (ranking, a per-expert scan of the counts, placement).  Every
// path writes the same tables: ids, renormalised weights and the shared-expert gate
// per token, the pairs bucketed by expert, and one 64-byte job record per used
// expert (expert, first position, count, 0, first 12 pair ids) so an expert
// workgroup learns everything about its job from one scalar load.
#include "device.h"
#include "internal.h"
#include "routing.h"

namespace moeffn {

constexpr int kRouterWaves = 4;
constexpr int kRouterTile = 8;  // most tokens per workgroup column

// Sums eight values over the wave in one transposed butterfly: each exchange keeps
// half of the values in each half of its lane group and adds the partner's copy, so
// after the swaps across halves (permlane32), across rows of 16 (permlane16) and across
// the two 8-lane halves of a row (a row rotation by 8) every lane holds a partial sum of
// one value, tok = lane bits 32, 16, 8 read as 4, 2, 1; the 8 lanes that share tok then
// finish the sum inside their group.  Each step adds two partial sums that are the same
// in both lanes of a pair, so all 8 lanes end with identical bits.
__device__ __forceinline__ float seg_sum8(const float (&a)[8], int lane, int &tok) {
    const bool h3 = (lane & 8) != 0;
    float b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = swap32_add(a[i], a[i + 4]);        // halves keep i / i + 4
    const float c0 = swap16_add(b[0], b[2]), c1 = swap16_add(b[1], b[3]);  // rows keep 0 / 2
    const float send = h3 ? c0 : c1, keep = h3 ? c1 : c0;
    float v = keep + dpp_f<kDppRowRor8>(send);
    v = v + dpp_f<kDppHalfMirror>(v);
    v = v + dpp_f<kDppXor2>(v);
    v = v + dpp_f<kDppXor1>(v);
    tok = ((lane & 32) ? 4 : 0) + ((lane & 16) ? 2 : 0) + (h3 ? 1 : 0);
    return v;
}

// One workgroup per row (E router rows, then the gate vector as row E) and token
// tile: the four waves split the row into quarters, so the E+1 rows spread over
// every CU and each lane issues only its few 16-byte loads.  Lane l of wave w holds
// chunks w*CPW + l + 64n (n < NC) of the fp32 row.
template <int NC, bool XBF>
__global__ __launch_bounds__(256) void k_router(RouterParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ float s_part[kRouterWaves][2][kRouterTile];  // per wave: dot products, squares
    __shared__ float s_rho[kRouterTile];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = p.H, E = p.E;
    const int n_chunks = H / 4;            // fp32 rows, 4 elements per 16-byte chunk
    const int cpw = n_chunks / kRouterWaves;  // chunks per wave (H is a multiple of 32)
    const int row = blockIdx.x;
    const float *W = row < E ? p.router + (size_t)row * H : p.gate_vec;

    float4 w[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int q = lane + 64 * n;
        w[n] = q < cpw ? *reinterpret_cast<const float4 *>(W + 4 * (wave * cpw + q))
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // input RMSNorm folded into the dot products: logit = rho * sum_h (W[h] * g[h]) * x[h],
    // rho = 1/sqrt(mean(x^2) + eps), the squares summed alongside (the same lanes and
    // order in every workgroup, so every workgroup gets the same rho bits).  The norm
    // weights are fetched with the rows and folded in once the tokens are staged, so
    // that no load waits for another
    const bool norm = p.norm_w != nullptr;
    float4 gn[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int q = lane + 64 * n;
        gn[n] = (norm && q < cpw) ? *reinterpret_cast<const float4 *>(p.norm_w + 4 * (wave * cpw + q))
                                  : make_float4(1.f, 1.f, 1.f, 1.f);
    }

    const int t0 = blockIdx.y * p.tok_tile;
    const int nt = min(p.tok_tile, p.T - t0);
    // the normalised tokens of the tile are written by the column's first workgroups,
    // one 4-element chunk per thread and pass; the first chunk's norm weights are
    // fetched now as well
    const int xn_units = norm ? nt * n_chunks : 0;
    const int xn_u0 = blockIdx.x * 256 + tid;
    float4 g0 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (xn_u0 < xn_units) g0 = *reinterpret_cast<const float4 *>(p.norm_w + 4 * (xn_u0 % n_chunks));
    const int xrow = H * (XBF ? 2 : 4);
    const uint8_t *xs = (const uint8_t *)p.x + (size_t)t0 * xrow;
    {
        // the tile is at most kStageBytes: 8 chunks per thread; a tile of at most one chunk
        // per thread (a single token of up to 2048 bf16 elements) issues one load, not eight
        // (a branch on a value all threads of the workgroup share)
        const int n16 = nt * xrow / 16;
        auto stage = [&](auto NQ) {
            constexpr int Q = decltype(NQ)::value;
            uint4 xv[Q];
            load_chunks<Q>(xv, n16, tid, [&](int i) { return xs + 16 * (size_t)i; });
#pragma unroll
            for (int q = 0; q < Q; ++q)
                if (tid + 256 * q < n16) reinterpret_cast<uint4 *>(lds)[tid + 256 * q] = xv[q];
        };
        if (n16 <= 256) stage(std::integral_constant<int, 1>{});
        else stage(std::integral_constant<int, 8>{});
    }
    __syncthreads();
    if (norm) {
#pragma unroll
        for (int n = 0; n < NC; ++n)
            w[n] = make_float4(w[n].x * gn[n].x, w[n].y * gn[n].y, w[n].z * gn[n].z, w[n].w * gn[n].w);
    }

    auto x_chunk = [&](int i, int c) -> float4 {
        if constexpr (XBF) {
            const uint2 b = *reinterpret_cast<const uint2 *>(lds + i * xrow + 8 * c);
            return make_float4(bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y));
        } else {
            return *reinterpret_cast<const float4 *>(lds + i * xrow + 16 * c);
        }
    };

    // partial dot products of up to 8 tokens, one transposed reduction per wave for all,
    // then the four quarters summed in wave order
    float acc[kRouterTile], ss[kRouterTile];
#pragma unroll
    for (int i = 0; i < kRouterTile; ++i) acc[i] = ss[i] = 0.f;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int q = lane + 64 * n;
        if (q < cpw) {
            const int c = wave * cpw + q;
#pragma unroll
            for (int i = 0; i < kRouterTile; ++i) {
                if (i < nt) {
                    const float4 xv = x_chunk(i, c);
                    acc[i] = fmaf(w[n].x, xv.x, acc[i]);
                    acc[i] = fmaf(w[n].y, xv.y, acc[i]);
                    acc[i] = fmaf(w[n].z, xv.z, acc[i]);
                    acc[i] = fmaf(w[n].w, xv.w, acc[i]);
                    if (norm) {
                        ss[i] = fmaf(xv.x, xv.x, ss[i]);
                        ss[i] = fmaf(xv.y, xv.y, ss[i]);
                        ss[i] = fmaf(xv.z, xv.z, ss[i]);
                        ss[i] = fmaf(xv.w, xv.w, ss[i]);
                    }
                }
            }
        }
    }
    int tok = 0;
    const float sum = seg_sum8(acc, lane, tok);
    const float sq = norm ? seg_sum8(ss, lane, tok) : 0.f;
    if ((lane & 7) == 0) {
        s_part[wave][0][tok] = sum;
        s_part[wave][1][tok] = sq;
    }
    __syncthreads();
    if (tid < nt) {
        float v = ((s_part[0][0][tid] + s_part[1][0][tid]) + s_part[2][0][tid]) + s_part[3][0][tid];
        float rho = 1.f;
        if (norm) {
            const float q = ((s_part[0][1][tid] + s_part[1][1][tid]) + s_part[2][1][tid]) + s_part[3][1][tid];
            rho = 1.0f / sqrtf(q / (float)H + p.norm_eps);
            v *= rho;
            s_rho[tid] = rho;
        }
        p.logits[(size_t)(t0 + tid) * logit_stride(E) + row] = v;
    }
    if (norm && blockIdx.x * 256 < xn_units) {
        // the normalised tokens, (x * rho) * g, that feed both expert branches, rounded
        // to the activation storage
        __syncthreads();
        for (int q = xn_u0; q < xn_units; q += 256 * gridDim.x) {
            const int i = q / n_chunks, c = q - i * n_chunks;
            const float r = s_rho[i];
            const float4 xv = x_chunk(i, c);
            const float4 g = q == xn_u0 ? g0 : *reinterpret_cast<const float4 *>(p.norm_w + 4 * c);
            const float v0 = __fmul_rn(__fmul_rn(xv.x, r), g.x), v1 = __fmul_rn(__fmul_rn(xv.y, r), g.y);
            const float v2 = __fmul_rn(__fmul_rn(xv.z, r), g.z), v3 = __fmul_rn(__fmul_rn(xv.w, r), g.w);
            const size_t o = (size_t)(t0 + i) * H + 4 * c;
            if constexpr (XBF) {
                uint2 b;
                b.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v0) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v1) << 16);
                b.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v2) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v3) << 16);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.xn) + o) = b;
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.xn) + o) = make_float4(v0, v1, v2, v3);
            }
        }
    }
}

// k_route: one workgroup, one wave per token (up to 16), ranks the batch and
// buckets it (5 to 16 tokens, and fewer where the gate/up workgroups cannot).
__global__ __launch_bounds__(1024) void k_route(RouterParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const RouteLds L = route_lds_layout(p.T, p.k, p.E, false);
    const RouteGlobal g{p.ids, p.wts, p.gate_s, p.records, p.n_unique, p.pairs, p.pos_expert,
                        p.dbg_ids, p.dbg_w, p.dbg_logits, p.dbg_gate};
    rank_tokens(p.logits, 0, p.T, p.E, p.k, lds, L, g);
    bucket_tokens(p.T, p.k, p.E, lds, L, g);
}

// ---- router GEMM for batches above 16 tokens ---------------------------------------------
// logits[t][e] = sum_h W[e][h] x[t][h] on v_mfma_f32_16x16x32_bf16.  The tokens are bf16;
// each fp32 router weight is split exactly into three bf16 pieces (hi = the top 16 bits,
// mid = the top 16 bits of the rest, lo = what remains, at most 8 significant bits), so
// every product piece * token is exact in fp32 and the three accumulate into one fp32
// sum: the logits carry fp32-GEMV accuracy.  A wave owns 16 rows (experts, the gate
// vector as row E), 16 * NT tokens and a quarter of K.  K in steps of 32; lane group g
// holds elements 8g..8g+7 of a step for both operands.
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rfloatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rfloatx4_t r_mfma(uint4 a, uint4 b, rfloatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rbf16x8_t, a),
                                                   __builtin_bit_cast(rbf16x8_t, b), c, 0, 0, 0);
}

// eight fp32 -> three bf16x8 planes whose sum is exact
__device__ __forceinline__ void split3(const float4 &u, const float4 &v, uint4 &hi, uint4 &mid, uint4 &lo) {
    const float f[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t b = __float_as_uint(f[i]);
        const float fh = __uint_as_float(b & 0xffff0000u);
        const float r1 = f[i] - fh;
        const uint32_t bm = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(bm);
        h[i] = b >> 16;
        m[i] = bm >> 16;
        l[i] = __float_as_uint(r2) >> 16;
    }
    hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    mid = make_uint4(m[0] | (m[1] << 16), m[2] | (m[3] << 16), m[4] | (m[5] << 16), m[6] | (m[7] << 16));
    lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}


// One K step (32 elements) of a wave: its 16 weight rows (8 fp32 per lane) and its
// token tiles (8 bf16 per lane each).  Steps are loaded two ahead in three register
// sets; the main loop loads unconditionally (clamped rows and tokens are read and
// never stored) so that each wait counts only the loads issued after the one it needs.
template <int NT>  // 16-token tiles per wave (each workgroup: 16 * NT tokens)
struct RgStep {
    float4 wa, wb;
    uint4 b[NT];
};

// A workgroup owns 16 rows and 16 * NT tokens, and its four waves split K in quarters
// (workgroups of 64 rows over the whole of K left most of the GPU idle below a few
// thousand tokens and were slower at every size measured); the partial sums meet in
// LDS and wave 0 adds them in wave order (((w0 + w1) + w2) + w3) and stores the logits.
template <int NT>
__global__ __launch_bounds__(256) void k_router_mfma(RouterParams p) {
    constexpr int kRgTiles = NT, kRgTokens = 16 * NT;
    __shared__ float s_part[3][kRgTiles][4][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ri = lane & 15, g = lane >> 4;
    const int H = p.H, E = p.E, T = p.T;
    const int row = blockIdx.x * 16 + ri;  // A row of this lane (rows past E read the gate vector)
    const float *W = (row < E ? p.router + (size_t)row * H : p.gate_vec) + 8 * g;
    const int t0 = blockIdx.y * kRgTokens;
    const uint16_t *xb[kRgTiles];
#pragma unroll
    for (int n = 0; n < kRgTiles; ++n) {
        const int t = t0 + 16 * n + ri;
        xb[n] = reinterpret_cast<const uint16_t *>(p.x) + (size_t)(t < T ? t : 0) * H + 8 * g;
    }
    rfloatx4_t acc[kRgTiles];
#pragma unroll
    for (int n = 0; n < kRgTiles; ++n) acc[n] = rfloatx4_t{0.f, 0.f, 0.f, 0.f};
    // this wave's steps: s0 .. s0 + per - 1 (H is a multiple of 128, so per >= 1); loads
    // past the last step re-read the last one and are never used
    const int per = H / 128, s0 = wave * per;
    RgStep<NT> st[3];
    auto load = [&](RgStep<NT> &d, int s) {
        const int ko = 32 * (s0 + min(s, per - 1));
        d.wa = *reinterpret_cast<const float4 *>(W + ko);
        d.wb = *reinterpret_cast<const float4 *>(W + ko + 4);
#pragma unroll
        for (int n = 0; n < kRgTiles; ++n) d.b[n] = ld16(xb[n] + ko);
    };
    auto mul = [&](const RgStep<NT> &d) {
        uint4 hi, mid, lo;
        split3(d.wa, d.wb, hi, mid, lo);
#pragma unroll
        for (int n = 0; n < kRgTiles; ++n) {
            acc[n] = r_mfma(hi, d.b[n], acc[n]);
            acc[n] = r_mfma(mid, d.b[n], acc[n]);
            acc[n] = r_mfma(lo, d.b[n], acc[n]);
        }
    };
    load(st[0], 0);
    load(st[1], 1);
    int s = 0;
    for (; s + 4 < per; s += 3) {
        load(st[2], s + 2); mul(st[0]);
        load(st[0], s + 3); mul(st[1]);
        load(st[1], s + 4); mul(st[2]);
    }
    if (s + 2 < per) load(st[2], s + 2);
    mul(st[0]);
    if (s + 1 < per) { if (s + 3 < per) load(st[0], s + 3); mul(st[1]); }
    if (s + 2 < per) mul(st[2]);
    if (s + 3 < per) mul(st[0]);
    if (wave > 0) {
#pragma unroll
        for (int n = 0; n < kRgTiles; ++n)
#pragma unroll
            for (int v = 0; v < 4; ++v) s_part[wave - 1][n][v][lane] = acc[n][v];
    }
    lds_barrier();
    if (wave != 0) return;
    // lane holds rows 4g + v of the workgroup's 16 for token column ri
#pragma unroll
    for (int n = 0; n < kRgTiles; ++n) {
        const int t = t0 + 16 * n + ri;
        if (t >= T) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int e = blockIdx.x * 16 + 4 * g + v;
            const float sum = ((acc[n][v] + s_part[0][n][v][lane]) + s_part[1][n][v][lane]) + s_part[2][n][v][lane];
            if (e <= E) p.logits[(size_t)t * logit_stride(E) + e] = sum;
        }
    }
}

// The same GEMM for thousands of tokens, with rows split over the waves instead of K: a
// workgroup owns 16 * NT tokens and every row (the E experts and the gate vector, in
// 16-row tiles; wave w takes tiles w, w + 4, ..., at most RTW of them) over the whole
// of K.  Each token row is then read once per workgroup (the four waves' loads of the
// same token bytes meet in the L1) instead of once per 16 rows, and each weight is split
// into its three pieces once per workgroup of 64 tokens instead of once per 16.  Each
// logit is one accumulator over K in ascending 32-element steps.
template <int RTW, int NT>
__global__ __launch_bounds__(256) void k_router_mfma_rows(RouterParams p) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it
    const int ri = lane & 15, g = lane >> 4;
    const int H = p.H, E = p.E, T = p.T;
    const int n_tiles = (E + 1 + 15) / 16;
    int nt = 0;  // this wave's row tiles
#pragma unroll
    for (int i = 0; i < RTW; ++i) nt += wave + 4 * i < n_tiles ? 1 : 0;
    if (nt == 0) return;
    const float *W[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int row = (wave + 4 * i) * 16 + ri;  // rows past E read the gate vector, never stored
        W[i] = (row < E ? p.router + (size_t)row * H : p.gate_vec) + 8 * g;
    }
    const int t0 = blockIdx.x * 16 * NT;
    const uint16_t *xb[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int t = t0 + 16 * n + ri;
        xb[n] = reinterpret_cast<const uint16_t *>(p.x) + (size_t)(t < T ? t : 0) * H + 8 * g;
    }
    rfloatx4_t acc[RTW][NT];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[i][n] = rfloatx4_t{0.f, 0.f, 0.f, 0.f};
    struct Step {
        float4 wa[RTW], wb[RTW];
        uint4 b[NT];
    };
    const int nsteps = H / 32;
    // loads past the last step re-read the last one and are never used; the tiles a wave
    // does not own re-read its first tile (uniform per wave, so no divergence)
    auto load = [&](Step &d, int s) {
        const int ko = 32 * min(s, nsteps - 1);
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const float *w = (i < nt ? W[i] : W[0]) + ko;
            d.wa[i] = *reinterpret_cast<const float4 *>(w);
            d.wb[i] = *reinterpret_cast<const float4 *>(w + 4);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) d.b[n] = ld16(xb[n] + ko);
    };
    auto mul = [&](const Step &d) {
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            if (i >= nt) break;
            uint4 hi, mid, lo;
            split3(d.wa[i], d.wb[i], hi, mid, lo);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                acc[i][n] = r_mfma(hi, d.b[n], acc[i][n]);
                acc[i][n] = r_mfma(mid, d.b[n], acc[i][n]);
                acc[i][n] = r_mfma(lo, d.b[n], acc[i][n]);
            }
        }
    };
    Step st[3];
    load(st[0], 0);
    load(st[1], 1);  // H is a multiple of 128: at least four steps
    int s = 0;
    for (; s + 4 < nsteps; s += 3) {
        load(st[2], s + 2); mul(st[0]);
        load(st[0], s + 3); mul(st[1]);
        load(st[1], s + 4); mul(st[2]);
    }
    if (s + 2 < nsteps) load(st[2], s + 2);
    mul(st[0]);
    if (s + 1 < nsteps) { if (s + 3 < nsteps) load(st[0], s + 3); mul(st[1]); }
    if (s + 2 < nsteps) mul(st[2]);
    if (s + 3 < nsteps) mul(st[0]);
    // lane holds rows 16 * tile + 4g + v for token column ri
    const int ls = logit_stride(E);
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        if (i >= nt) break;
        const int e0 = (wave + 4 * i) * 16 + 4 * g;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int t = t0 + 16 * n + ri;
            if (t >= T) continue;
            float *dst = p.logits + (size_t)t * ls + e0;
            if (e0 + 3 <= E) {
                *reinterpret_cast<float4 *>(dst) = make_float4(acc[i][n][0], acc[i][n][1], acc[i][n][2], acc[i][n][3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (e0 + v <= E) dst[v] = acc[i][n][v];
            }
        }
    }
}

// row split used from this many tokens (below, the K-split kernel fills more of the GPU)
constexpr int kRouterRowsMinTokens = 8192;
constexpr int kRouterRowsRTW = 5, kRouterRowsNT = 4;

hipError_t launch_router_mfma(const RouterParams &p, hipStream_t s) {
    if (!p.x_bf16 || p.norm_w || p.H % 128 != 0) return hipErrorInvalidValue;
    // one 16-token tile per workgroup up to 256 tokens; wider token blocks above (fewer
    // re-reads and splits of the rows)
    const int n_tiles = (p.E + 1 + 15) / 16;
    if (p.T >= kRouterRowsMinTokens && n_tiles > 4 * (kRouterRowsRTW - 1) && n_tiles <= 4 * kRouterRowsRTW) {
        const int tpw = 16 * kRouterRowsNT;
        launch_kernel(k_router_mfma_rows<kRouterRowsRTW, kRouterRowsNT>, dim3((p.T + tpw - 1) / tpw), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    const int nt = p.T <= 256 ? 1 : p.T < 4096 ? 2 : 4;
    const dim3 grid((p.E + 1 + 15) / 16, (p.T + 16 * nt - 1) / (16 * nt));
    if (nt == 1) launch_kernel(k_router_mfma<1>, grid, dim3(256), 0, s, p);
    else if (nt == 2) launch_kernel(k_router_mfma<2>, grid, dim3(256), 0, s, p);
    else launch_kernel(k_router_mfma<4>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---- batch routing (large batches) ----------------------------------------------------
// Three launches, no atomics, a deterministic result: buckets hold their pairs in pair
// order, as the one-workgroup bucketing of smaller batches does.
//   k_rank_batch    a workgroup ranks a group of tokens (one wave per token in turn),
//                   writes its row of per-expert counts and, per pair, the
//                   number of earlier pairs of the workgroup with the same expert;
//   k_count_scan    per expert, the exclusive prefix of the count rows (in place) and
//                   the expert's total;
//   k_bucket_batch  every workgroup scans the totals (expert offsets, used-expert
//                   slots); workgroup 0 writes the job records; each pair goes to
//                   offset + prefix of its workgroup + its rank inside the workgroup.
// A ranking workgroup takes 4 tokens (one per wave) up to 4096 tokens and 16 (four per
// wave in turn) above, where more count rows would cost the scan more than the
// parallel ranking saves.
// bcount layout (ints): totals [E], then the count rows [W][E] (W = ceil(T / tokens per
// ranking workgroup)), then the in-workgroup ranks [T*k].
constexpr int kRankTokensPerWaveMax = 4;
constexpr int kRankPairsMax = 4 * kRankTokensPerWaveMax * kMaxTopK;

static __host__ __device__ int rank_tokens_per_wave(int T) { return T > 4096 ? 4 : 1; }
static __host__ __device__ int rank_tokens_per_wg(int T) { return 4 * rank_tokens_per_wave(T); }

__global__ __launch_bounds__(256) void k_rank_batch(RouterParams p) {
    __shared__ int s_ids[kRankPairsMax];
    __shared__ int s_hist[kMaxExperts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = p.E, k = p.k;
    const int tpw = rank_tokens_per_wave(p.T);
    const int tw0 = blockIdx.x * 4 * tpw;
    const int ntw = min(4 * tpw, p.T - tw0);
    for (int e = tid; e < E; e += 256) s_hist[e] = 0;
    for (int i = 0; i < tpw; ++i) {
        const int lt = i * 4 + wave, t = tw0 + lt;
        if (lt >= ntw) break;
        RouteOut o{p.ids + (size_t)t * k, p.wts + (size_t)t * k, p.gate_s + t,
                   p.dbg_ids ? p.dbg_ids + (size_t)t * k : nullptr, p.dbg_w ? p.dbg_w + (size_t)t * k : nullptr,
                   p.dbg_gate ? p.dbg_gate + t : nullptr, p.dbg_logits ? p.dbg_logits + (size_t)t * E : nullptr};
        route_token_any(p.logits + (size_t)t * logit_stride(E), E, k, lane, o);
        if (lane < k) s_ids[lt * k + lane] = o.ids[lane];  // this lane's own store
    }
    __syncthreads();
    const int np = ntw * k;
    int *rank = p.bcount + E + (size_t)gridDim.x * E;
    for (int q = tid; q < np; q += 256) {
        const int e = s_ids[q];
        int r = 0;
        for (int j = 0; j < q; ++j) r += s_ids[j] == e ? 1 : 0;
        rank[(size_t)tw0 * k + q] = r;
        if (e >= 0 && e < E) atomicAdd(&s_hist[e], 1);  // LDS: exact whatever the order
    }
    __syncthreads();
    int *row = p.bcount + E + (size_t)blockIdx.x * E;
    for (int e = tid; e < E; e += 256) row[e] = s_hist[e];
}

// one workgroup per expert: exclusive prefix of its column over the W count rows
__global__ __launch_bounds__(256) void k_count_scan(RouterParams p, int W) {
    __shared__ int s_wsum[4];
    const int e = blockIdx.x, E = p.E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int *col = p.bcount + E + e;
    const int per = (W + 255) / 256, w0 = tid * per;
    int a = 0;
    for (int i = 0; i < per; ++i)
        if (w0 + i < W) a += col[(size_t)(w0 + i) * E];
    const int ia = wave_incl_scan(a, lane);
    if (lane == 63) s_wsum[wave] = ia;
    __syncthreads();
    int base = ia - a;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    for (int i = 0; i < per; ++i)
        if (w0 + i < W) {
            int *c = col + (size_t)(w0 + i) * E;
            const int v = *c;
            *c = base;
            base += v;
        }
    if (tid == 255) p.bcount[e] = base;  // the last thread ends on the total
}

constexpr int kBucketPairsPerWg = 1024;

__global__ __launch_bounds__(256) void k_bucket_batch(RouterParams p) {
    __shared__ int s_off[kMaxExperts], s_slot[kMaxExperts], s_wsum[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = p.E, NP = p.T * p.k, k = p.k;
    const int *cnt = p.bcount;
    const int *pre = p.bcount + E;
    const int tpg = rank_tokens_per_wg(p.T);
    const int W = (p.T + tpg - 1) / tpg;
    const int *rank = p.bcount + E + (size_t)W * E;
    // exclusive scans of cnt[] and (cnt[] > 0): thread owns two consecutive experts
    const int e0 = 2 * tid;
    const int c0 = e0 < E ? cnt[e0] : 0, c1 = e0 + 1 < E ? cnt[e0 + 1] : 0;
    int a = c0 + c1, b = (c0 > 0) + (c1 > 0);
    const int ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
    if (lane == 63) { s_wsum[0][wave] = ia; s_wsum[1][wave] = ib; }
    __syncthreads();
    int ba = ia - a, bb = ib - b;
    for (int w = 0; w < wave; ++w) { ba += s_wsum[0][w]; bb += s_wsum[1][w]; }
    if (e0 < E) { s_off[e0] = ba; s_slot[e0] = c0 > 0 ? bb : -1; }
    if (e0 + 1 < E) { s_off[e0 + 1] = ba + c0; s_slot[e0 + 1] = c1 > 0 ? bb + (c0 > 0) : -1; }
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int e = tid; e < E; e += 256) {
            const int u = s_slot[e];
            if (u < 0) continue;
            const int c = cnt[e];
            int *rec = p.records + (size_t)u * kRecInts;
            rec[0] = e; rec[1] = s_off[e]; rec[2] = c; rec[3] = 0;
            for (int f = c; f < kRecPairs; ++f) rec[4 + f] = -1;  // the pairs themselves come below
        }
        if (tid == 0) *p.n_unique = s_wsum[1][0] + s_wsum[1][1] + s_wsum[1][2] + s_wsum[1][3];
    }
    const int q_end = min(NP, (blockIdx.x + 1) * kBucketPairsPerWg);
    for (int q = blockIdx.x * kBucketPairsPerWg + tid; q < q_end; q += 256) {
        const int e = p.ids[q];
        if (e < 0 || e >= E) continue;
        const int w = (q / k) / tpg;
        const int r = pre[(size_t)w * E + e] + rank[q];  // place inside the expert's bucket
        const int pos = s_off[e] + r;
        if (r >= cnt[e] || pos >= NP) continue;  // only with corrupt counts
        p.pairs[pos] = q;
        p.pos_expert[pos] = e;
        if (r < kRecPairs) p.records[(size_t)s_slot[e] * kRecInts + 4 + r] = q;
    }
}

size_t batch_route_ints(int T, int k, int E) {
    // the most count rows any batch up to T tokens needs
    const size_t W = T > 4096 ? std::max<size_t>(1024, ((size_t)T + 15) / 16) : ((size_t)T + 3) / 4;
    return (size_t)E + W * E + (size_t)T * k;
}

hipError_t launch_rank_batch(const RouterParams &p, hipStream_t s) {
    const int grid = (p.T + rank_tokens_per_wg(p.T) - 1) / rank_tokens_per_wg(p.T);
    if (p.k > kMaxTopK || p.E > kMaxExperts) return hipErrorInvalidValue;
    launch_kernel(k_rank_batch, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_count_scan(const RouterParams &p, hipStream_t s) {
    const int W = (p.T + rank_tokens_per_wg(p.T) - 1) / rank_tokens_per_wg(p.T);
    launch_kernel(k_count_scan, dim3(p.E), dim3(256), 0, s, p, W);
    return hipGetLastError();
}

hipError_t launch_bucket_batch(const RouterParams &p, hipStream_t s) {
    if (p.E > 2 * 256) return hipErrorInvalidValue;
    const int grid = (p.T * p.k + kBucketPairsPerWg - 1) / kBucketPairsPerWg;
    launch_kernel(k_bucket_batch, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

int route_kernel_waves(int T) { return T < 4 ? 4 : T > 16 ? 16 : T; }

size_t route_kernel_lds_bytes(int T, int k, int E) {
    return route_lds_layout(T, k, E, false).bytes;
}

hipError_t launch_route(const RouterParams &p, hipStream_t s) {
    const size_t lds = route_kernel_lds_bytes(p.T, p.k, p.E);
    if (lds > kLdsLimit) return hipErrorInvalidValue;
    launch_kernel(k_route, dim3(1), dim3(64 * route_kernel_waves(p.T)), lds, s, p);
    return hipGetLastError();
}

size_t router_lds_bytes(const RouterParams &p) {
    return (size_t)p.tok_tile * p.H * (p.x_bf16 ? 2 : 4);
}

template <int NC>
static hipError_t launch_router_t(const RouterParams &p, int grid_tiles, hipStream_t s) {
    const size_t lds = router_lds_bytes(p);
    const dim3 grid(p.E + 1, grid_tiles);
    if (p.x_bf16)
        launch_kernel(k_router<NC, true>, grid, dim3(256), lds, s, p);
    else
        launch_kernel(k_router<NC, false>, grid, dim3(256), lds, s, p);
    return hipGetLastError();
}

int router_chunks_per_lane(int H) {
    const int per_wave = H / 4 / kRouterWaves;
    int nc = 1;
    while (64 * nc < per_wave) nc <<= 1;
    return nc;
}

hipError_t launch_router(const RouterParams &p, int grid_tiles, hipStream_t s) {
    if (router_lds_bytes(p) > kStageBytes || p.tok_tile > kRouterTile || p.H % 32 != 0) return hipErrorInvalidValue;
    switch (router_chunks_per_lane(p.H)) {
    case 1: return launch_router_t<1>(p, grid_tiles, s);
    case 2: return launch_router_t<2>(p, grid_tiles, s);
    case 4: return launch_router_t<4>(p, grid_tiles, s);
    case 8: return launch_router_t<8>(p, grid_tiles, s);
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

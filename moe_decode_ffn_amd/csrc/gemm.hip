// gemm.hip -- grouped MFMA GEMM for the larger-batch regime (bf16 weights).
//
// At batch 128 each used expert sees ~4 tokens and every expert's weights are
// still read once, so the layer stays HBM-bound; the MFMA path is here because
// the per-expert work is now a real [n_e x K] x [K x rows] contraction.
//
// Tiling: a wave owns 16 weight rows (the MFMA M side) and up to 16*NT tokens
// of the job's expert (N side, 16 per tile, zero-padded), K in chunks of 128.
// A job is 64 rows (four waves) of one expert; a routed job walks its whole
// bucket in passes of 16*NT tokens, a shared-expert job owns one block of
// 16*NT tokens, so the shared expert spreads over (row tiles x token blocks).
// v_mfma_f32_16x16x32_bf16 takes 8 bf16 of A and 8 of B per lane from the same
// K slot (lane group g = lane/16); a sum over K does not care which K slot
// holds which element as long as A and B agree.  So in MFMA step s of a
// 128-element chunk, lane group g holds elements s*32 + g*8 .. +7: one 16-byte
// load per lane, and the four groups of a row read 64 contiguous bytes per
// load instruction.  Token rows are read the same way.
// Result D[i][j] of a 16x16 tile sits in lane 16*(i/4) + j, element i%4.
//
// k_gg_gate_up: h = silu(gate . x) * (up . x), stored bf16 (the down GEMM's
//   operand), per (token, slot) pair; shared expert: per token.
// k_gg_down:    y = down . h per pair (fp32), S = shared_down . h_s; the join
//   kernel of the mat-vec path finishes the layer.
#include "device.h"
#include "internal.h"

namespace moeffn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kGGWaves = 4;
constexpr int kGGRows = 16 * kGGWaves;  // weight rows per job
constexpr int kGGChunk = 128;           // K elements per chunk (four MFMA steps)

int gg_rows_per_job() { return kGGRows; }

__device__ __forceinline__ floatx4_t mfma16(uint4 a, uint4 b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// round to nearest even bf16 (the compiler's conversion; a hardware instruction on gfx950)
__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

struct GGJob {
    bool valid, routed;
    const uint8_t *W0, *W1;
    int K, rows, tile, ntok;
    int tok0;            // shared expert: first token of the job's block
    const int *rec;
};

// Jobs: the shared expert's (row tile, token block) pairs first, token blocks
// of tb_len tokens, then tiles_routed row tiles per used expert.
__device__ __forceinline__ GGJob gg_decode(int j, int tiles_shared, int tb_len, int tiles_routed,
                                           int nu, const int *records, int E, int npairs,
                                           const uint8_t *rW0, const uint8_t *rW1, int rrows, int rK,
                                           const uint8_t *sW0, const uint8_t *sW1, int srows, int sK,
                                           int T) {
    GGJob jb{};
    jb.valid = false;
    const int n_tb = (T + tb_len - 1) / tb_len;
    if (j < tiles_shared * n_tb) {
        const int tb = j / tiles_shared;
        jb.valid = true; jb.routed = false;
        jb.W0 = sW0; jb.W1 = sW1; jb.K = sK; jb.rows = srows; jb.tile = j - tb * tiles_shared;
        jb.tok0 = tb * tb_len;
        jb.ntok = min(tb_len, T - jb.tok0);
        jb.rec = nullptr;
        return jb;
    }
    j -= tiles_shared * n_tb;
    const int slot = j / tiles_routed;
    if (slot >= nu) return jb;
    const int *rec = records + (size_t)slot * kRecInts;
    const int e = rec[0], start = rec[1], cnt = rec[2];
    if (e < 0 || e >= E || start < 0 || cnt <= 0 || start + cnt > npairs) return jb;
    jb.valid = true; jb.routed = true;
    const size_t m0 = (size_t)e * rrows * rK * 2;
    jb.W0 = rW0 + m0;
    jb.W1 = rW1 ? rW1 + m0 : nullptr;
    jb.K = rK; jb.rows = rrows; jb.tile = j - slot * tiles_routed; jb.ntok = cnt; jb.tok0 = 0;
    jb.rec = rec;
    return jb;
}

__device__ __forceinline__ int gg_pair(const int *rec, const int *pairs, int a) {
    return a < kRecPairs ? rec[4 + a] : pairs[rec[1] + a];
}

// the four 16-byte pieces of a bf16 row this lane feeds to the MFMA steps of one
// chunk: elements k0 + 32*s .. +7 for s = 0..3 (k0 = chunk start + 8*g)
__device__ __forceinline__ void ld_chunk(const uint8_t *row, int k0, bool ok, uint4 (&v)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
        v[s] = ok ? ld16(row + (size_t)(k0 + 32 * s) * 2) : make_uint4(0, 0, 0, 0);
}

// ---- gate/up --------------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void k_gg_gate_up(GGParams p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ri = lane & 15, g = lane >> 4;
    const int T = p.T, k = p.k, npairs = T * k;
    int nu = p.routed ? *p.n_unique : 0;
    nu = nu < 0 ? 0 : nu > p.E ? p.E : nu;
    const int J = p.tiles_shared * ((T + 16 * NT - 1) / (16 * NT)) + nu * p.tiles_routed;
    for (int j = blockIdx.x; j < J; j += gridDim.x) {
        const GGJob jb = gg_decode(j, p.tiles_shared, 16 * NT, p.tiles_routed, nu, p.records, p.E,
                                   npairs, p.w0, p.w1, p.I, p.H, p.sw0, p.sw1, p.Is, p.H, T);
        if (!jb.valid) continue;
        const int row = jb.tile * kGGRows + wave * 16 + ri;  // A row of this lane
        const bool rok = row < jb.rows;
        const size_t rb = (size_t)jb.K * 2;
        const uint8_t *arow0 = jb.W0 + (size_t)(rok ? row : 0) * rb;
        const uint8_t *arow1 = jb.W1 + (size_t)(rok ? row : 0) * rb;
        const int nchunk = jb.K / kGGChunk;
        for (int t0 = 0; t0 < jb.ntok; t0 += 16 * NT) {
            // token rows of this lane's columns (N side)
            const uint8_t *brow[NT];
            bool bok[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int a = t0 + 16 * n + ri;
                int tok = 0;
                bok[n] = a < jb.ntok;
                if (bok[n]) {
                    if (jb.routed) {
                        const int pr = gg_pair(jb.rec, p.pairs, a);
                        bok[n] = pr >= 0 && pr < npairs;
                        tok = bok[n] ? pr / k : 0;
                    } else {
                        tok = jb.tok0 + a;
                    }
                }
                brow[n] = (const uint8_t *)p.x + (size_t)tok * p.H * 2;
            }
            floatx4_t accg[NT], accu[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                accg[n] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                accu[n] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            }
            uint4 a0[4], a1[4], b[NT][4], na0[4], na1[4], nb[NT][4];
            ld_chunk(arow0, g * 8, rok, a0);
            ld_chunk(arow1, g * 8, rok, a1);
#pragma unroll
            for (int n = 0; n < NT; ++n) ld_chunk(brow[n], g * 8, bok[n], b[n]);
            for (int c = 0; c < nchunk; ++c) {
                const bool more = c + 1 < nchunk;
                const int kn = (c + 1) * kGGChunk + g * 8;
                if (more) {
                    ld_chunk(arow0, kn, rok, na0);
                    ld_chunk(arow1, kn, rok, na1);
#pragma unroll
                    for (int n = 0; n < NT; ++n) ld_chunk(brow[n], kn, bok[n], nb[n]);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        accg[n] = mfma16(a0[s], b[n][s], accg[n]);
                        accu[n] = mfma16(a1[s], b[n][s], accu[n]);
                    }
                if (more) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        a0[s] = na0[s];
                        a1[s] = na1[s];
#pragma unroll
                        for (int n = 0; n < NT; ++n) b[n][s] = nb[n][s];
                    }
                }
            }
            // epilogue: lane holds rows 4*g + v of the tile, token column ri
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int a = t0 + 16 * n + ri;
                if (a >= jb.ntok) continue;
                int orow = jb.tok0 + a;
                if (jb.routed) {
                    orow = gg_pair(jb.rec, p.pairs, a);
                    if (orow < 0 || orow >= npairs) continue;
                }
                uint16_t *dst = reinterpret_cast<uint16_t *>(jb.routed ? (uintptr_t)p.hb : (uintptr_t)p.shb);
                const int stride = jb.routed ? p.I : p.Is;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = jb.tile * kGGRows + wave * 16 + 4 * g + v;
                    if (r < jb.rows)
                        dst[(size_t)orow * stride + r] = to_bf16(silu_f(accg[n][v]) * accu[n][v]);
                }
            }
        }
    }
}

// ---- down -------------------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void k_gg_down(GGParams p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ri = lane & 15, g = lane >> 4;
    const int T = p.T, k = p.k, npairs = T * k, H = p.H;
    int nu = p.routed ? *p.n_unique : 0;
    nu = nu < 0 ? 0 : nu > p.E ? p.E : nu;
    const int J = p.tiles_shared * ((T + 16 * NT - 1) / (16 * NT)) + nu * p.tiles_routed;
    for (int j = blockIdx.x; j < J; j += gridDim.x) {
        const GGJob jb = gg_decode(j, p.tiles_shared, 16 * NT, p.tiles_routed, nu, p.records, p.E,
                                   npairs, p.w0, nullptr, H, p.I, p.sw0, nullptr, H, p.Is, T);
        if (!jb.valid) continue;
        const int row = jb.tile * kGGRows + wave * 16 + ri;
        const bool rok = row < jb.rows;
        const size_t rb = (size_t)jb.K * 2;
        const uint8_t *arow = jb.W0 + (size_t)(rok ? row : 0) * rb;
        const int nchunk = jb.K / kGGChunk;
        const uint8_t *hbase = reinterpret_cast<const uint8_t *>(jb.routed ? (uintptr_t)p.hb : (uintptr_t)p.shb);
        for (int t0 = 0; t0 < jb.ntok; t0 += 16 * NT) {
            const uint8_t *brow[NT];
            bool bok[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int a = t0 + 16 * n + ri;
                int src = 0;
                bok[n] = a < jb.ntok;
                if (bok[n]) {
                    if (jb.routed) {
                        const int pr = gg_pair(jb.rec, p.pairs, a);
                        bok[n] = pr >= 0 && pr < npairs;
                        src = bok[n] ? pr : 0;
                    } else {
                        src = jb.tok0 + a;
                    }
                }
                brow[n] = hbase + (size_t)src * rb;
            }
            floatx4_t acc[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            uint4 a0[4], b[NT][4], na0[4], nb[NT][4];
            ld_chunk(arow, g * 8, rok, a0);
#pragma unroll
            for (int n = 0; n < NT; ++n) ld_chunk(brow[n], g * 8, bok[n], b[n]);
            for (int c = 0; c < nchunk; ++c) {
                const bool more = c + 1 < nchunk;
                const int kn = (c + 1) * kGGChunk + g * 8;
                if (more) {
                    ld_chunk(arow, kn, rok, na0);
#pragma unroll
                    for (int n = 0; n < NT; ++n) ld_chunk(brow[n], kn, bok[n], nb[n]);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[n] = mfma16(a0[s], b[n][s], acc[n]);
                if (more) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        a0[s] = na0[s];
#pragma unroll
                        for (int n = 0; n < NT; ++n) b[n][s] = nb[n][s];
                    }
                }
            }
            float *dst = reinterpret_cast<float *>(jb.routed ? (uintptr_t)p.y : (uintptr_t)p.S);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int a = t0 + 16 * n + ri;
                if (a >= jb.ntok) continue;
                int orow = jb.tok0 + a;
                if (jb.routed) {
                    orow = gg_pair(jb.rec, p.pairs, a);
                    if (orow < 0 || orow >= npairs) continue;
                }
                const int r0 = jb.tile * kGGRows + wave * 16 + 4 * g;
                if (r0 + 3 < jb.rows) {
                    *reinterpret_cast<float4 *>(dst + (size_t)orow * H + r0) =
                        make_float4(acc[n][0], acc[n][1], acc[n][2], acc[n][3]);
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (r0 + v < jb.rows) dst[(size_t)orow * H + r0 + v] = acc[n][v];
                }
            }
        }
    }
}

hipError_t launch_gg_gate_up(const GGParams &p, int nt, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (nt <= 1) launch_kernel(k_gg_gate_up<1>, dim3(grid), dim3(256), 0, s, p);
    else if (nt <= 2) launch_kernel(k_gg_gate_up<2>, dim3(grid), dim3(256), 0, s, p);
    else launch_kernel(k_gg_gate_up<4>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gg_down(const GGParams &p, int nt, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (nt <= 1) launch_kernel(k_gg_down<1>, dim3(grid), dim3(256), 0, s, p);
    else if (nt <= 2) launch_kernel(k_gg_down<2>, dim3(grid), dim3(256), 0, s, p);
    else launch_kernel(k_gg_down<4>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

int gg_occupancy(bool gate_up, int nt) {
    int n = 0;
    hipError_t e;
    if (gate_up)
        e = nt <= 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gg_gate_up<1>, 256, 0)
          : nt <= 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gg_gate_up<2>, 256, 0)
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gg_gate_up<4>, 256, 0);
    else
        e = nt <= 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gg_down<1>, 256, 0)
          : nt <= 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gg_down<2>, 256, 0)
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gg_down<4>, 256, 0);
    return e == hipSuccess && n > 0 ? n : 1;
}

}  // namespace moeffn

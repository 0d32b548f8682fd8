// prefill.hip -- grouped MFMA GEMM for large batches (prefill chunks).
//
// With thousands of tokens every expert holds a bucket of ~T*k/E tokens, so a
// job's weight tile is worth sharing across many tokens.  A job is 128 weight
// rows of one expert (gate/up: 64 rows of gate and the same 64 rows of up, so
// that silu(gate) * up is formed in registers; down: 128 rows), and a pass
// covers 16*NW*NTW tokens of its bucket: each of the NW waves owns 16*NTW of
// the pass's tokens and all 128 rows.  128- and 192-token passes run four waves
// (one a SIMD, NTW 2 and 3); 256-token passes run eight waves of 32 tokens, two
// a SIMD, whose registers fit in half the file (four waves of 64 tokens need more
// than half, so one a SIMD, with nothing to run while it waits).  K runs in
// stages of 64:
//   * the weight stage (128 rows x 128 bytes) is loaded once per workgroup into
//     LDS (double-buffered; 16-byte chunk c of row r sits at chunk position
//     c ^ (r & 7), so the fragment reads hit distinct banks) and read by all the
//     waves;
//   * each wave loads its own token rows straight into registers; loads run two
//     stages ahead in three register sets, and the barriers between stages order
//     LDS only, so the prefetched loads stay in flight across them;
//   * per 32-element K step a wave runs 8 x NTW v_mfma_f32_16x16x32_bf16.
// The K order and the lane-to-K mapping are those of the smaller grouped GEMM
// (32-element steps in ascending order, lane group g holding elements 8g..8g+7
// of a step), so the two give the same bits.
// Outputs as in the smaller GEMM: h in bf16 per (token, slot) pair or shared
// token, y / S in fp32.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace moeffn {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kPfRows = 128;                        // weight rows per job
constexpr int kPfBK = 64;                           // K elements per stage
constexpr int kPfStride = kPfBK * 2;                // LDS bytes per weight row
constexpr int kPfStage = kPfRows * kPfStride;       // LDS bytes per stage

__device__ __forceinline__ floatx4_t pf_mfma(uint4 a, uint4 b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

struct PfJob {
    bool valid, routed;
    const uint8_t *W0, *W1;  // gate/up: gate and up matrices; down: the matrix (W1 unused)
    int K, rows, tile;       // reduction length, rows of the matrix, row tile
    int ntok, tok0;          // tokens of the job; shared expert: first token of its block
    int start;               // routed: first bucketed position of the expert
};

// Jobs: the shared expert's (row tile, token block) pairs first, then the row
// tiles of every used expert (each walks its whole bucket in passes).  Every job of
// one token block or one expert runs on one XCD, so that the tokens its row tiles
// all read come from that XCD's L2: with workgroups dispatched round-robin over the
// 8 XCDs and a grid that is a multiple of 8, job j runs on XCD j % 8, and job j
// belongs to block (or expert) 8 * (j / 8 / tiles) + j % 8, row tile (j / 8) % tiles.
__host__ __device__ inline int pf_round8(int v) { return (v + 7) & ~7; }

__host__ __device__ inline int pf_jobs(int tiles_shared, int n_tb, int nu, int tiles_routed) {
    return tiles_shared * pf_round8(n_tb) + pf_round8(nu) * tiles_routed;
}

template <bool GU>
__device__ __forceinline__ PfJob pf_decode(const GGParams &p, int j, int tb_len, int nu, int npairs) {
    PfJob jb{};
    jb.valid = false;
    const int n_tb = (p.T + tb_len - 1) / tb_len;
    const int shared_jobs = p.tiles_shared * pf_round8(n_tb);
    if (j < shared_jobs) {
        const int x = j & 7, r = j >> 3;
        const int tb = 8 * (r / p.tiles_shared) + x;
        if (tb >= n_tb) return jb;
        jb.valid = true;
        jb.routed = false;
        jb.W0 = p.sw0;
        jb.W1 = p.sw1;
        jb.K = GU ? p.H : p.Is;
        jb.rows = GU ? p.Is : p.H;
        jb.tile = r % p.tiles_shared;
        jb.tok0 = tb * tb_len;
        jb.ntok = min(tb_len, p.T - jb.tok0);
        jb.start = 0;
        return jb;
    }
    j -= shared_jobs;
    const int x = j & 7, r = j >> 3;
    const int slot = 8 * (r / p.tiles_routed) + x;
    if (slot >= nu) return jb;
    const int *rec = p.records + (size_t)slot * kRecInts;
    const int e = rec[0], start = rec[1], cnt = rec[2];
    if (e < 0 || e >= p.E || start < 0 || cnt <= 0 || start + cnt > npairs) return jb;
    const int rows = GU ? p.I : p.H, K = GU ? p.H : p.I;
    const size_t m0 = (size_t)e * rows * K * 2;
    jb.valid = true;
    jb.routed = true;
    jb.W0 = p.w0 + m0;
    jb.W1 = GU ? p.w1 + m0 : nullptr;
    jb.K = K;
    jb.rows = rows;
    jb.tile = r % p.tiles_routed;
    jb.ntok = cnt;
    jb.tok0 = 0;
    jb.start = start;
    return jb;
}

template <bool GU, int NTW, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_pf(GGParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int BN = 16 * NW * NTW;  // tokens per pass
    constexpr int NQ = 16 / NW;        // 16-byte weight chunks per thread per stage
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ri = lane & 15, g = lane >> 4;
    const int T = p.T, k = p.k, npairs = T * k;
    int nu = p.routed ? *p.n_unique : 0;
    nu = nu < 0 ? 0 : nu > p.E ? p.E : nu;
    const int J = pf_jobs(p.tiles_shared, (T + BN - 1) / BN, nu, p.tiles_routed);
    // rows of the tile as a gate/up job sees them: 64 of gate, then the same 64 of up
    constexpr int kHalf = GU ? kPfRows / 2 : kPfRows;

    for (int j = blockIdx.x; j < J; j += gridDim.x) {
        const PfJob jb = pf_decode<GU>(p, j, BN, nu, npairs);
        if (!jb.valid) continue;
        const size_t rb = (size_t)jb.K * 2;
        const int nst = jb.K / kPfBK;
        // this thread's 16-byte pieces of every weight stage (NQ of them): row u>>3, chunk u&7
        const uint8_t *asrc[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int u = tid + 64 * NW * q, lr = u >> 3, ch = u & 7;
            const int half = lr / kHalf, r = jb.tile * kHalf + (lr - half * kHalf);
            const uint8_t *W = half ? jb.W1 : jb.W0;
            asrc[q] = W + (size_t)(r < jb.rows ? r : 0) * rb + ch * 16;
        }
        const uint8_t *bbase = GU ? (const uint8_t *)p.x
                                  : (const uint8_t *)(jb.routed ? (const void *)p.hb : (const void *)p.shb);

        for (int t0 = 0; t0 < jb.ntok; t0 += BN) {
            // this lane's token rows (B side) and output rows, one per 16-token tile
            const uint8_t *brow[NTW];
            int orow[NTW];
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                const int a = t0 + wave * 16 * NTW + 16 * n + ri;
                int src = 0, o = -1;
                if (a < jb.ntok) {
                    if (jb.routed) {
                        const int pr = p.pairs[jb.start + a];
                        const bool ok = pr >= 0 && pr < npairs;
                        o = ok ? pr : -1;
                        src = ok ? (GU ? pr / k : pr) : 0;
                    } else {
                        o = jb.tok0 + a;
                        src = o;
                    }
                }
                orow[n] = o;
                brow[n] = bbase + (size_t)src * rb;
            }

            floatx4_t acc[8][NTW];
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int n = 0; n < NTW; ++n) acc[m][n] = floatx4_t{0.f, 0.f, 0.f, 0.f};

            // three register sets in rotation: stage s is loaded two stages ahead, its
            // weights go to LDS slot s % 2 one stage ahead, its tokens feed the MFMAs
            uint4 areg[3][NQ], breg[3][NTW][2];
            auto load = [&](auto SI, int st) {
                constexpr int i = decltype(SI)::value;
                const size_t ko = (size_t)st * kPfBK * 2;
                // unconditional (branch-free) loads: rows past the end read a clamped row,
                // and the epilogue stores neither their rows nor their token columns
#pragma unroll
                for (int q = 0; q < NQ; ++q) areg[i][q] = ld16(asrc[q] + ko);
#pragma unroll
                for (int n = 0; n < NTW; ++n)
#pragma unroll
                    for (int s = 0; s < 2; ++s) breg[i][n][s] = ld16(brow[n] + ko + (size_t)(32 * s + 8 * g) * 2);
            };
            auto stash = [&](auto SI, int st) {  // weights of stage st into LDS slot st % 2
                constexpr int i = decltype(SI)::value;
                uint8_t *dst = lds + (st & 1) * kPfStage;
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int u = tid + 64 * NW * q;
                    *reinterpret_cast<uint4 *>(dst + (u >> 3) * kPfStride + (((u & 7) ^ ((u >> 3) & 7)) << 4)) = areg[i][q];
                }
            };
            // one stage: prefetch stage st + 2, multiply stage st, stash stage st + 1.  The
            // main loop issues its loads unconditionally so that the compiler's wait before
            // each use counts only the loads issued after it (a conditional load makes it
            // wait for all of them); the last few stages go through the guarded tail.
            auto body = [&](auto SI, int st, bool fetch, bool keep) {
                constexpr int i = decltype(SI)::value;
                if (fetch) load(std::integral_constant<int, (i + 2) % 3>{}, st + 2);
                const uint8_t *cur = lds + (st & 1) * kPfStage;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    uint4 a[8];
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        a[m] = *reinterpret_cast<const uint4 *>(cur + (16 * m + ri) * kPfStride +
                                                                (((4 * s + g) ^ ((16 * m + ri) & 7)) << 4));
#pragma unroll
                    for (int n = 0; n < NTW; ++n)
#pragma unroll
                        for (int m = 0; m < 8; ++m) acc[m][n] = pf_mfma(a[m], breg[i][n][s], acc[m][n]);
                }
                if (keep) stash(std::integral_constant<int, (i + 1) % 3>{}, st + 1);
                lds_barrier();
            };
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            lds_barrier();  // every wave is done with both LDS slots (previous pass or job)
            load(I0{}, 0);
            load(I1{}, 1);  // K is a multiple of 128: at least two stages
            stash(I0{}, 0);
            lds_barrier();
            int st = 0;
            for (; st + 4 < nst; st += 3) {
                body(I0{}, st, true, true);
                body(I1{}, st + 1, true, true);
                body(I2{}, st + 2, true, true);
            }
            // tail: at most four stages, set index continuing from st % 3 == 0
            body(I0{}, st, st + 2 < nst, st + 1 < nst);
            if (st + 1 < nst) body(I1{}, st + 1, st + 3 < nst, st + 2 < nst);
            if (st + 2 < nst) body(I2{}, st + 2, st + 4 < nst, st + 3 < nst);
            if (st + 3 < nst) body(I0{}, st + 3, false, false);

            // epilogue: lane holds rows 16m + 4g + v of the tile for token column ri
            if constexpr (GU) {
                uint16_t *dst = jb.routed ? p.hb : p.shb;
                const int stride = jb.routed ? p.I : p.Is;
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    if (orow[n] < 0) continue;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int r = jb.tile * kHalf + 16 * m + 4 * g;
                        if (r + 3 >= jb.rows) continue;
                        uint32_t w2[2];
#pragma unroll
                        for (int v = 0; v < 4; v += 2) {
                            const float h0 = silu_f(acc[m][n][v]) * acc[m + 4][n][v];
                            const float h1 = silu_f(acc[m][n][v + 1]) * acc[m + 4][n][v + 1];
                            w2[v / 2] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)h0) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)h1) << 16);
                        }
                        *reinterpret_cast<uint2 *>(dst + (size_t)orow[n] * stride + r) = make_uint2(w2[0], w2[1]);
                    }
                }
            } else {
                float *dst = jb.routed ? p.y : p.S;
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    if (orow[n] < 0) continue;
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const int r = jb.tile * kPfRows + 16 * m + 4 * g;
                        if (r + 3 >= jb.rows) continue;
                        *reinterpret_cast<float4 *>(dst + (size_t)orow[n] * p.H + r) =
                            make_float4(acc[m][n][0], acc[m][n][1], acc[m][n][2], acc[m][n][3]);
                    }
                }
            }
        }
    }
}

}  // namespace

size_t pf_lds_bytes() { return 2 * (size_t)kPfStage; }
int pf_job_count(int tiles_shared, int n_tb, int nu, int tiles_routed) {
    return pf_jobs(tiles_shared, n_tb, nu, tiles_routed);
}
int pf_rows_per_job(bool gate_up) { return gate_up ? kPfRows / 2 : kPfRows; }
int pf_tokens_per_pass(int ntw) { return 64 * ntw; }  // ntw 4: eight waves of 32 tokens

hipError_t launch_pf(const GGParams &p, bool gate_up, int ntw, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    const size_t lds = pf_lds_bytes();
    if (gate_up) {
        if (ntw <= 2) launch_kernel(k_pf<true, 2>, dim3(grid), dim3(256), lds, s, p);
        else if (ntw == 3) launch_kernel(k_pf<true, 3>, dim3(grid), dim3(256), lds, s, p);
        else launch_kernel(k_pf<true, 2, 8>, dim3(grid), dim3(512), lds, s, p);
    } else {
        if (ntw <= 2) launch_kernel(k_pf<false, 2>, dim3(grid), dim3(256), lds, s, p);
        else if (ntw == 3) launch_kernel(k_pf<false, 3>, dim3(grid), dim3(256), lds, s, p);
        else launch_kernel(k_pf<false, 2, 8>, dim3(grid), dim3(512), lds, s, p);
    }
    return hipGetLastError();
}

int pf_occupancy(bool gate_up, int ntw) {
    int n = 0;
    const size_t lds = pf_lds_bytes();
    hipError_t e;
    if (gate_up)
        e = ntw <= 2   ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<true, 2>, 256, lds)
            : ntw == 3 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<true, 3>, 256, lds)
                       : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<true, 2, 8>, 512, lds);
    else
        e = ntw <= 2   ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<false, 2>, 256, lds)
            : ntw == 3 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<false, 3>, 256, lds)
                       : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<false, 2, 8>, 512, lds);
    return e == hipSuccess && n > 0 ? n : 1;
}

}  // namespace moeffn

// prefill.hip -- grouped MFMA GEMM for large batches (prefill chunks).
//
// With thousands of tokens every expert holds a bucket of ~T*k/E tokens, so a
// job's weight tile is worth sharing across many tokens.  A job is 128 weight
// rows of one expert (gate/up: 64 rows of gate and the same 64 rows of up, so
// that silu(gate) * up is formed in registers; down: 128 rows), and a pass
// covers 64*NTW tokens of its bucket: each of the four waves owns 16*NTW of
// the pass's tokens and all 128 rows.  K runs in stages of 64:
//   * the weight stage (128 rows x 128 bytes) is loaded once per workgroup into
//     LDS (double-buffered, rows padded to 144 bytes so the fragment reads hit
//     distinct banks) and read by all four waves;
//   * each wave loads its own token rows straight into registers, one stage
//     ahead;
//   * per 32-element K step a wave runs 8 x NTW v_mfma_f32_16x16x32_bf16.
// The K order and the lane-to-K mapping are those of the smaller grouped GEMM
// (32-element steps in ascending order, lane group g holding elements 8g..8g+7
// of a step), so the two give the same bits.
// Outputs as in the smaller GEMM: h in bf16 per (token, slot) pair or shared
// token, y / S in fp32.
#include "device.h"
#include "internal.h"

namespace moeffn {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kPfRows = 128;                        // weight rows per job
constexpr int kPfBK = 64;                           // K elements per stage
constexpr int kPfStride = kPfBK * 2 + 16;           // LDS bytes per weight row (padded)
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
// tiles of every used expert (each walks its whole bucket in passes).
template <bool GU>
__device__ __forceinline__ PfJob pf_decode(const GGParams &p, int j, int tb_len, int nu, int npairs) {
    PfJob jb{};
    jb.valid = false;
    const int n_tb = (p.T + tb_len - 1) / tb_len;
    if (j < p.tiles_shared * n_tb) {
        const int tb = j / p.tiles_shared;
        jb.valid = true;
        jb.routed = false;
        jb.W0 = p.sw0;
        jb.W1 = p.sw1;
        jb.K = GU ? p.H : p.Is;
        jb.rows = GU ? p.Is : p.H;
        jb.tile = j - tb * p.tiles_shared;
        jb.tok0 = tb * tb_len;
        jb.ntok = min(tb_len, p.T - jb.tok0);
        jb.start = 0;
        return jb;
    }
    j -= p.tiles_shared * n_tb;
    const int slot = j / p.tiles_routed;
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
    jb.tile = j - slot * p.tiles_routed;
    jb.ntok = cnt;
    jb.tok0 = 0;
    jb.start = start;
    return jb;
}

template <bool GU, int NTW>
__global__ __launch_bounds__(256) void k_pf(GGParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int BN = 64 * NTW;  // tokens per pass
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ri = lane & 15, g = lane >> 4;
    const int T = p.T, k = p.k, npairs = T * k;
    int nu = p.routed ? *p.n_unique : 0;
    nu = nu < 0 ? 0 : nu > p.E ? p.E : nu;
    const int J = p.tiles_shared * ((T + BN - 1) / BN) + nu * p.tiles_routed;
    // rows of the tile as a gate/up job sees them: 64 of gate, then the same 64 of up
    constexpr int kHalf = GU ? kPfRows / 2 : kPfRows;

    for (int j = blockIdx.x; j < J; j += gridDim.x) {
        const PfJob jb = pf_decode<GU>(p, j, BN, nu, npairs);
        if (!jb.valid) continue;
        const size_t rb = (size_t)jb.K * 2;
        const int nst = jb.K / kPfBK;
        // this thread's four 16-byte pieces of every weight stage: row u>>3, chunk u&7
        const uint8_t *asrc[4];
        bool aok[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int u = tid + 256 * q, lr = u >> 3, ch = u & 7;
            const int half = lr / kHalf, r = jb.tile * kHalf + (lr - half * kHalf);
            aok[q] = r < jb.rows;
            const uint8_t *W = half ? jb.W1 : jb.W0;
            asrc[q] = W + (size_t)(aok[q] ? r : 0) * rb + ch * 16;
        }
        const uint8_t *bbase = GU ? (const uint8_t *)p.x
                                  : (const uint8_t *)(jb.routed ? (const void *)p.hb : (const void *)p.shb);

        for (int t0 = 0; t0 < jb.ntok; t0 += BN) {
            // this lane's token rows (B side) and output rows, one per 16-token tile
            const uint8_t *brow[NTW];
            bool bok[NTW];
            int orow[NTW];
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                const int a = t0 + wave * 16 * NTW + 16 * n + ri;
                bok[n] = a < jb.ntok;
                int src = 0, o = -1;
                if (bok[n]) {
                    if (jb.routed) {
                        const int pr = p.pairs[jb.start + a];
                        bok[n] = pr >= 0 && pr < npairs;
                        o = bok[n] ? pr : -1;
                        src = bok[n] ? (GU ? pr / k : pr) : 0;
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

            // stage 0: weights to LDS buffer 0, tokens to registers
            uint4 areg[4], b[NTW][2], nb[NTW][2];
#pragma unroll
            for (int q = 0; q < 4; ++q) areg[q] = aok[q] ? ld16(asrc[q]) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    b[n][s] = bok[n] ? ld16(brow[n] + (size_t)(32 * s + 8 * g) * 2) : make_uint4(0, 0, 0, 0);
            __syncthreads();  // the previous pass's readers are done with both buffers
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = tid + 256 * q;
                *reinterpret_cast<uint4 *>(lds + (u >> 3) * kPfStride + (u & 7) * 16) = areg[q];
            }
            __syncthreads();

            for (int st = 0; st < nst; ++st) {
                const bool more = st + 1 < nst;
                const uint8_t *cur = lds + (st & 1) * kPfStage;
                if (more) {
                    const size_t ko = (size_t)(st + 1) * kPfBK * 2;
#pragma unroll
                    for (int q = 0; q < 4; ++q) areg[q] = aok[q] ? ld16(asrc[q] + ko) : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int n = 0; n < NTW; ++n)
#pragma unroll
                        for (int s = 0; s < 2; ++s)
                            nb[n][s] = bok[n] ? ld16(brow[n] + ko + (size_t)(32 * s + 8 * g) * 2)
                                              : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    uint4 a[8];
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        a[m] = *reinterpret_cast<const uint4 *>(cur + (16 * m + ri) * kPfStride + (32 * s + 8 * g) * 2);
#pragma unroll
                    for (int n = 0; n < NTW; ++n)
#pragma unroll
                        for (int m = 0; m < 8; ++m) acc[m][n] = pf_mfma(a[m], b[n][s], acc[m][n]);
                }
                if (more) {
                    uint8_t *nxt = lds + ((st + 1) & 1) * kPfStage;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int u = tid + 256 * q;
                        *reinterpret_cast<uint4 *>(nxt + (u >> 3) * kPfStride + (u & 7) * 16) = areg[q];
                    }
#pragma unroll
                    for (int n = 0; n < NTW; ++n) {
                        b[n][0] = nb[n][0];
                        b[n][1] = nb[n][1];
                    }
                }
                __syncthreads();
            }

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
int pf_rows_per_job(bool gate_up) { return gate_up ? kPfRows / 2 : kPfRows; }
int pf_tokens_per_pass(int ntw) { return 64 * ntw; }

hipError_t launch_pf(const GGParams &p, bool gate_up, int ntw, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    const size_t lds = pf_lds_bytes();
    if (gate_up) {
        if (ntw <= 2) launch_kernel(k_pf<true, 2>, dim3(grid), dim3(256), lds, s, p);
        else launch_kernel(k_pf<true, 4>, dim3(grid), dim3(256), lds, s, p);
    } else {
        if (ntw <= 2) launch_kernel(k_pf<false, 2>, dim3(grid), dim3(256), lds, s, p);
        else launch_kernel(k_pf<false, 4>, dim3(grid), dim3(256), lds, s, p);
    }
    return hipGetLastError();
}

int pf_occupancy(bool gate_up, int ntw) {
    int n = 0;
    const size_t lds = pf_lds_bytes();
    hipError_t e;
    if (gate_up)
        e = ntw <= 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<true, 2>, 256, lds)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<true, 4>, 256, lds);
    else
        e = ntw <= 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<false, 2>, 256, lds)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_pf<false, 4>, 256, lds);
    return e == hipSuccess && n > 0 ? n : 1;
}

}  // namespace moeffn

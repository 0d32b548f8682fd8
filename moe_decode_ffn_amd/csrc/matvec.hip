// matvec.hip -- small-batch (mat-vec regime) expert kernels.
//
// Work is cut into jobs: one job = one expert (a used routed expert, or the
// shared expert) x one tile of that expert's rows.  Routed jobs exist only for
// the experts the batch actually selected (the used-expert count is read on
// the device), so every expert's weights are streamed once per call whatever
// the number of tokens that chose it.  Each workgroup walks jobs with a grid
// stride and issues the next job's 16-byte weight loads before it computes the
// current one, so HBM stays busy across job boundaries; per job it needs one
// scalar read of the job record (expert, tokens) and no other dependent load.
//
// k_gate_up: h = silu(gate . x) * (up . x) per (token, slot) pair; the batch's
//   tokens are staged in LDS once (or per pass when they do not fit).
// k_down:    y = down . h per pair (routed) and S = shared_down . h_s (shared),
//   one expert per job.
// k_join:    out = sum_j w_j y_j (slot order) + s * S, product and sum rounded
//   separately.
// k_down_join: down + join in one launch for small batches: a workgroup of 16
//   waves owns a tile of output rows for every pair, keeps y in LDS and joins.
// Storage: fp32, bf16, or 4-bit blocks (32 elements + one fp16 scale per block,
// dequantised in registers).
#include <algorithm>
#include <type_traits>

#include "device.h"
#include "internal.h"
#include "routing.h"

namespace moeffn {

constexpr int kWaves = 4;

template <int WK> struct WTraits;
template <> struct WTraits<W_F32> { static constexpr int epc = 4, rpw_gu = 1, rpw_d = 2; };
template <> struct WTraits<W_BF16> { static constexpr int epc = 8, rpw_gu = 2, rpw_d = 4; };
template <> struct WTraits<W_Q4> { static constexpr int epc = 32, rpw_gu = 2, rpw_d = 4; };

static int rpw_gu_of(int wk) {
    return wk == W_F32 ? WTraits<W_F32>::rpw_gu : wk == W_BF16 ? WTraits<W_BF16>::rpw_gu
                                                              : WTraits<W_Q4>::rpw_gu;
}
static int rpw_d_of(int wk) {
    return wk == W_F32 ? WTraits<W_F32>::rpw_d : wk == W_BF16 ? WTraits<W_BF16>::rpw_d
                                                             : WTraits<W_Q4>::rpw_d;
}

// A bf16 single token routed inside the gate/up workgroups reads one row per wave per job
// instead of two: twice the jobs over more resident workgroups, so the last round of jobs
// is a smaller part of the launch (from 2 tokens on, the two-row jobs, which read each
// staged token once for two rows, are as fast or faster).
bool gate_up_one_row(int wkind, const RowMap &m, int T, bool route_here) {
    return wkind == W_BF16 && m.lpr == 64 && T == 1 && route_here;
}
int gate_up_rows_per_wg(int wkind, const RowMap &m, int T, bool route_here) {
    return kWaves * (gate_up_one_row(wkind, m, T, route_here) ? 1 : rpw_gu_of(wkind)) * (64 / m.lpr);
}
int down_rows_per_wg(int wkind, const RowMap &m) { return kWaves * rpw_d_of(wkind) * (64 / m.lpr); }

template <int WK>
__device__ __forceinline__ size_t row_bytes(int k) {
    return WK == W_F32 ? (size_t)k * 4 : WK == W_BF16 ? (size_t)k * 2 : (size_t)k / 2;
}

// pair id of the a-th token of a routed job: inline in a 16-int job record up to
// kRecPairs (INL), else from the bucketed pairs at the job's first position
template <bool INL>
__device__ __forceinline__ int job_pair(const int *rec, const int *pairs, int a) {
    if constexpr (INL) return a < kRecPairs ? rec[4 + a] : pairs[rec[1] + a];
    return pairs[rec[1] + a];
}

// ---- chunk dot products ------------------------------------------------------------------

// bf16 weights . bf16 activations (8 elements), fp32 accumulate
__device__ __forceinline__ float dot_bf16_bf16(uint4 w, uint4 x, float acc) {
    acc = dot2_bf16(w.x, x.x, acc);
    acc = dot2_bf16(w.y, x.y, acc);
    acc = dot2_bf16(w.z, x.z, acc);
    acc = dot2_bf16(w.w, x.w, acc);
    return acc;
}

// fp32 weights . fp32 activations (4 elements)
__device__ __forceinline__ float dot_f32_f32(uint4 w, float4 x, float acc) {
    acc = fmaf(__uint_as_float(w.x), x.x, acc);
    acc = fmaf(__uint_as_float(w.y), x.y, acc);
    acc = fmaf(__uint_as_float(w.z), x.z, acc);
    acc = fmaf(__uint_as_float(w.w), x.w, acc);
    return acc;
}

// bf16 weights . fp32 activations (8 elements)
__device__ __forceinline__ float dot_bf16_f32(uint4 w, float4 a0, float4 a1, float acc) {
    acc = fmaf(bf16_lo(w.x), a0.x, acc);
    acc = fmaf(bf16_hi(w.x), a0.y, acc);
    acc = fmaf(bf16_lo(w.y), a0.z, acc);
    acc = fmaf(bf16_hi(w.y), a0.w, acc);
    acc = fmaf(bf16_lo(w.z), a1.x, acc);
    acc = fmaf(bf16_hi(w.z), a1.y, acc);
    acc = fmaf(bf16_lo(w.w), a1.z, acc);
    acc = fmaf(bf16_hi(w.w), a1.w, acc);
    return acc;
}

// 4-bit block . bf16 activations in q4 pair order: sum_e (128 + u_e) x_e
__device__ __forceinline__ float dot_q4_bf16(uint4 w, const uint32_t xp[16]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t b[4];
        q4_word_to_bf16_pairs(ws[i], b);
        acc = dot2_bf16(b[0], xp[4 * i + 0], acc);
        acc = dot2_bf16(b[1], xp[4 * i + 1], acc);
        acc = dot2_bf16(b[2], xp[4 * i + 2], acc);
        acc = dot2_bf16(b[3], xp[4 * i + 3], acc);
    }
    return acc;
}

// 4-bit block . fp32 activations: sum_e u_e a_e (u = stored nibble)
__device__ __forceinline__ float dot_q4_f32(uint4 w, const float (&a)[32]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = ws[i] & 0x0f0f0f0fu, hi = (ws[i] >> 4) & 0x0f0f0f0fu;
        acc = fmaf((float)(lo & 0xffu), a[8 * i + 0], acc);
        acc = fmaf((float)(hi & 0xffu), a[8 * i + 1], acc);
        acc = fmaf((float)((lo >> 8) & 0xffu), a[8 * i + 2], acc);
        acc = fmaf((float)((hi >> 8) & 0xffu), a[8 * i + 3], acc);
        acc = fmaf((float)((lo >> 16) & 0xffu), a[8 * i + 4], acc);
        acc = fmaf((float)((hi >> 16) & 0xffu), a[8 * i + 5], acc);
        acc = fmaf((float)(lo >> 24), a[8 * i + 6], acc);
        acc = fmaf((float)(hi >> 24), a[8 * i + 7], acc);
    }
    return acc;
}

// Marks a loaded value as used (no instruction): the compiler waits for the load here.
__device__ __forceinline__ void consume(const uint4 &v) {
    asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}

// ---- jobs -----------------------------------------------------------------------------------
struct Job {
    bool valid, routed;
    const uint8_t *W0, *W1;   // weight matrices (gate, up) or (down, unused)
    const uint16_t *S0, *S1;  // 4-bit scales
    int K, rows, tile, ntok;
    const int *rec;           // routed: the job record
};

// Job j of a launch: shared tiles first, then tiles of used routed experts.  A used
// expert's entry in `records` is RI ints: (expert, first position, count, ...) -- a
// 16-int job record in memory, or a 4-int bucket slot in LDS.
template <int WK, int RI = kRecInts>
__device__ __forceinline__ Job decode_job(int j, int tiles_shared, int tiles_routed, int nu,
                                          const int *records, int E, int npairs,
                                          const uint8_t *rW0, const uint8_t *rW1,
                                          const uint16_t *rS0, const uint16_t *rS1, int rrows, int rK,
                                          const uint8_t *sW0, const uint8_t *sW1,
                                          const uint16_t *sS0, const uint16_t *sS1, int srows, int sK,
                                          int T) {
    Job jb{};
    jb.valid = false;
    if (j < tiles_shared) {
        jb.valid = true; jb.routed = false;
        jb.W0 = sW0; jb.W1 = sW1; jb.S0 = sS0; jb.S1 = sS1;
        jb.K = sK; jb.rows = srows; jb.tile = j; jb.ntok = T; jb.rec = nullptr;
        return jb;
    }
    j -= tiles_shared;
    const int slot = j / tiles_routed;
    if (slot >= nu) return jb;
    const int *rec = records + (size_t)slot * RI;
    const int e = rec[0], start = rec[1], cnt = rec[2];
    if (e < 0 || e >= E || start < 0 || cnt <= 0 || start + cnt > npairs) return jb;
    jb.valid = true; jb.routed = true;
    const size_t m0 = (size_t)e * rrows;
    const size_t rb = row_bytes<WK>(rK);
    jb.W0 = rW0 + m0 * rb;
    jb.W1 = rW1 ? rW1 + m0 * rb : nullptr;
    if constexpr (WK == W_Q4) {
        jb.S0 = rS0 + m0 * (rK / 32);
        jb.S1 = rS1 ? rS1 + m0 * (rK / 32) : nullptr;
    }
    jb.K = rK; jb.rows = rrows; jb.tile = j - slot * tiles_routed; jb.ntok = cnt; jb.rec = rec;
    return jb;
}

// Loads this lane's chunks of the job's rows (RPW rows per wave, NC chunks each).
// Every load is issued, whether or not the row or chunk exists: one that does not
// reads the job's first chunk (`safe` / `ssafe` for an invalid job) and its value is
// never used (rows past the job, chunks past the row and invalid jobs are skipped
// where the registers are consumed).  A fixed number of loads per call lets the
// compiler wait for exactly the loads a computation needs while the next job's are in
// flight; with conditional loads it would wait for every load issued before the use.
template <int WK, int LPR, int NC, int RPW, bool TWO>
__device__ __forceinline__ void load_rows(const Job &jb, int wave, int seg, int sl, uint4 (&w0)[RPW][NC],
                                          uint4 (&w1)[RPW][NC], float (&s0)[RPW][NC],
                                          float (&s1)[RPW][NC], const uint8_t *safe, const uint16_t *ssafe) {
    constexpr int RPI = 64 / LPR;
    constexpr int RPWG = kWaves * RPW * RPI;
    const size_t rb = row_bytes<WK>(jb.K);
    const int nch = (int)(rb / 16), nsb = jb.K / 32;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = jb.tile * RPWG + (wave * RPW + i) * RPI + seg;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const int c = sl + LPR * n;
            const bool ok = jb.valid && r < jb.rows && c < nch;
            // offsets inside one expert matrix: under 128 MiB where the planner accepts the
            // shapes (rows of at most 16 KiB, at most 8192 of them), so 32 bits for bf16 and
            // fp32 rows (fewer address instructions per load; 4-bit rows measured faster with
            // the 64-bit form)
            using OffT = std::conditional_t<WK == W_Q4, size_t, uint32_t>;
            const OffT off = ok ? (OffT)r * (OffT)rb + (OffT)16 * (OffT)c : (OffT)0;
            w0[i][n] = ld16(jb.valid ? jb.W0 + off : safe);
            if constexpr (TWO) w1[i][n] = ld16(jb.valid ? jb.W1 + off : safe);
            if constexpr (WK == W_Q4) {
                const size_t so = ok ? (size_t)r * nsb + c : 0;
                s0[i][n] = f16_to_f32(*(jb.valid ? jb.S0 + so : ssafe));
                if constexpr (TWO) s1[i][n] = f16_to_f32(*(jb.valid ? jb.S1 + so : ssafe));
            }
        }
    }
}

// ---- gate/up ------------------------------------------------------------------------------
template <int WK, int LPR, int NC, int RPW>
__device__ __forceinline__ void gate_up_token(const uint8_t *xr, const float *xbr, int n_chunks, int sl,
                                              const uint4 (&wg)[RPW][NC], const uint4 (&wu)[RPW][NC],
                                              const float (&sg)[RPW][NC], const float (&su)[RPW][NC],
                                              float (&g)[RPW], float (&u)[RPW]) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) { g[i] = 0.f; u[i] = 0.f; }
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = sl + LPR * n;
        if (c < n_chunks) {
            if constexpr (WK == W_BF16) {
                const uint4 xv = *reinterpret_cast<const uint4 *>(xr + 16 * c);
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    g[i] = dot_bf16_bf16(wg[i][n], xv, g[i]);
                    u[i] = dot_bf16_bf16(wu[i][n], xv, u[i]);
                }
            } else if constexpr (WK == W_F32) {
                const float4 xv = *reinterpret_cast<const float4 *>(xr + 16 * c);
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    g[i] = dot_f32_f32(wg[i][n], xv, g[i]);
                    u[i] = dot_f32_f32(wu[i][n], xv, u[i]);
                }
            } else {  // W_Q4: one 32-element block per chunk; the stage holds the token in
                      // the pair order of the weight decode and each block's bias 136 * sum x,
                      // so sum_e (128 + u_e) x_e - bias = sum_e q_e x_e
                uint32_t xp[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(xr + 64 * c + 16 * q);
                    xp[4 * q + 0] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
                }
                const float bias = xbr[c];
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    g[i] = fmaf(sg[i][n], dot_q4_bf16(wg[i][n], xp) - bias, g[i]);
                    u[i] = fmaf(su[i][n], dot_q4_bf16(wu[i][n], xp) - bias, u[i]);
                }
            }
        }
    }
}

// Bytes of the token stage: the tokens, and for 4-bit rows each block's bias after them.
__host__ __device__ inline size_t stage_x_bytes(int toks, int H, int xbytes) {
    return ((size_t)toks * H * xbytes + 15) & ~(size_t)15;
}
__host__ __device__ inline size_t stage_bytes(int toks, int H, int xbytes, int sums) {
    return stage_x_bytes(toks, H, xbytes) + (sums ? (((size_t)toks * (H / 32) * 4 + 15) & ~(size_t)15) : 0);
}

// Prefetch loads per thread (256 threads) for one token's row: a row of n chunks maps to
// LPR * NC >= n chunks of weights, and the token row is as many 16-byte chunks (4x for
// 4-bit rows, whose 32 elements take one chunk against four of bf16 tokens).  One token's
// logits row is at most 129 chunks (512 experts).
__host__ __device__ constexpr int one_token_x_loads(int wk, int lpr, int nc) {
    return ((wk == W_Q4 ? 4 : 1) * lpr * nc + 255) / 256 < 1 ? 1
           : ((wk == W_Q4 ? 4 : 1) * lpr * nc + 255) / 256 > 8 ? 8
                                                               : ((wk == W_Q4 ? 4 : 1) * lpr * nc + 255) / 256;
}
__host__ inline bool one_token_stage_fits(const GateUpParams &p, int wkind, const RowMap &m) {
    const size_t xb = wkind == W_F32 ? 4 : 2;
    return (size_t)p.H * xb / 16 <= 256 * (size_t)one_token_x_loads(wkind, m.lpr, m.nc) &&
           logit_stride(p.E) / 4 <= 256;
}

// RH: the workgroups rank and bucket the batch themselves (the job records then live
// in LDS; else in memory, written by a routing launch).  A compile-time choice, so
// that every record read has one known address space (a read through a pointer that
// may point to either is a flat load, which makes every later wait a wait for all
// outstanding memory operations).
// ONE: the launch serves a single token (the one-row variant always does).  SMALL: it
// serves 2 or more tokens with at most 64 (token, slot) pairs, which one wave buckets.
template <int WK, int LPR, int NC, bool RH, int RPWX = 0, bool ONE = (RPWX == 1), bool SMALL = false>
__global__ __launch_bounds__(256) void k_gate_up(GateUpParams p) {
    constexpr int RPW = RPWX ? RPWX : WTraits<WK>::rpw_gu;  // rows per wave per job
    constexpr int RPI = 64 / LPR;
    constexpr int RPWG = kWaves * RPW * RPI;
    constexpr int XB = WK == W_F32 ? 4 : 2;  // bytes per activation element
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, sl = lane % LPR;
    // a single-token instance (the one-row variant, and 4-bit rows routed here at batch 1)
    // has T = 1 at compile time: the batch paths (other tokens, bucketing) drop out, and
    // the scalar registers they held no longer spill
    const int H = p.H, T = ONE ? 1 : p.T, k = p.k;
    const int n_chunks = (int)(row_bytes<WK>(H) / 16);
    const int npairs = T * k;
    const size_t xrow = (size_t)H * XB;
    if constexpr (ONE || SMALL) {
        // the arguments a job's decode reads, fetched with the kernel's first scalar loads
        // rather than where the first job is decoded, after the routing barrier (measured
        // faster for batches of 1-8 tokens, slower for the general instances at 16)
        asm volatile("" ::"s"(p.wg), "s"(p.wu), "s"(p.I), "s"(p.swg), "s"(p.swu), "s"(p.Is));
        if constexpr (WK == W_Q4) asm volatile("" ::"s"(p.sg), "s"(p.su), "s"(p.ssg), "s"(p.ssu));
    }
    // 4-bit rows: each block's activation bias, after the staged tokens
    float *xbias = reinterpret_cast<float *>(lds + stage_x_bytes(p.x_resident ? T : p.tok_per_pass, H, XB));
    const int nblk = H / 32;
    // chunk i of the stage (16 bytes of one token's row; a block is 4 chunks held by 4
    // neighbouring lanes, which execute together): 4-bit rows keep the chunk in the
    // pair order of the weight decode, and the block's first lane writes its bias
    auto stage_store = [&](int i, uint4 v, bool ok) {
        if constexpr (WK == W_Q4) {
            const uint32_t xw[4] = {v.x, v.y, v.z, v.w};
            uint32_t xp[4];
            bf16x8_to_q4_order(xw, xp);
            float sx = ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
                       ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
            sx = sx + dpp_f<kDppXor1>(sx);
            sx = sx + dpp_f<kDppXor2>(sx);
            if (ok) {
                reinterpret_cast<uint4 *>(lds)[i] = make_uint4(xp[0], xp[1], xp[2], xp[3]);
                if ((i & 3) == 0) xbias[i >> 2] = 136.0f * sx;  // (128 + 8) * sum x
            }
        } else {
            if (ok) reinterpret_cast<uint4 *>(lds)[i] = v;
        }
    };
    // routing tables: global (routed by the router launch) or this workgroup's LDS
    const int *recs = p.records, *prs = p.pairs;
    int nu = 0;
    int j = blockIdx.x;
    auto decode = [&](int jj) {
        return decode_job<WK, RH ? 4 : kRecInts>(jj, p.tiles_shared, p.tiles_routed, nu, recs, p.E, npairs, p.wg, p.wu,
                              p.sg, p.su, p.I, H, p.swg, p.swu, p.ssg, p.ssu, p.Is, H, T);
    };
    uint4 ag[RPW][NC], au[RPW][NC], bg[RPW][NC], bu[RPW][NC];
    float asg[RPW][NC], asu[RPW][NC], bsg[RPW][NC], bsu[RPW][NC];
    Job ja{}, jb{};
    bool loaded = false;
    constexpr bool route_here = RH;
    // Loads go out in the order their data is needed (memory returns them in issue
    // order): the batch's logits rows when routing here (at most 5 16-byte chunks per
    // thread, e.g. 16 tokens of 256 experts), then the tokens resident in the stage (at most
    // kStageBytes: 8 chunks per thread), then the first job's weights.  Logits and tokens
    // reach LDS together before the routing, so that nothing between the bucketing and the
    // first computation waits for a load (a barrier that also waited for memory would hold
    // back the first job's weight loads and, behind them, the second job's).
    // a single-token instance loads only what one token can need (one_token_x_loads)
    constexpr int kLgPre = ONE ? 1 : 5, kXPre = ONE ? one_token_x_loads(WK, LPR, NC) : 8;
    const int n16lg = route_here ? T * logit_stride(p.E) / 4 : 0;
    uint4 lgpre[kLgPre];
    load_chunks<kLgPre>(lgpre, n16lg, tid, [&](int i) { return reinterpret_cast<const uint8_t *>(p.logits) + 16 * (size_t)i; });
    const int n16 = p.x_resident ? (int)(T * xrow / 16) : 0;
    uint4 xpre[kXPre];
    load_chunks<kXPre>(xpre, n16, tid, [&](int i) { return (const uint8_t *)p.x + 16 * (size_t)i; });
    if (!route_here) {
        nu = p.routed ? *p.n_unique : 0;
        nu = nu < 0 ? 0 : nu > p.E ? p.E : nu;
        if (j >= p.tiles_shared + nu * p.tiles_routed) return;
    }
    if (!route_here) {
        ja = decode(j);
        load_rows<WK, LPR, NC, RPW, true>(ja, wave, seg, sl, ag, au, asg, asu, p.swg, p.ssg);
        loaded = true;
    }
    if (route_here) {
        // every workgroup ranks and buckets the whole batch; workgroup 0 publishes
        uint8_t *area = lds + p.route_lds_off;
        const RouteLds L = route_lds_layout(T, k, p.E, true);
        float *lgt = reinterpret_cast<float *>(area + L.lgt);
#pragma unroll
        for (int q = 0; q < kLgPre; ++q)
            if (tid + 256 * q < n16lg) reinterpret_cast<uint4 *>(lgt)[tid + 256 * q] = lgpre[q];
        if (p.x_resident) {
#pragma unroll
            for (int q = 0; q < kXPre; ++q) stage_store(tid + 256 * q, xpre[q], tid + 256 * q < n16);
        }
        // every prefetch register counts as consumed here on every path (its stores above are
        // conditional): otherwise the compiler treats an unused one as still loading and, when
        // it reuses that register later, waits for every load issued since -- the first job's
        // weights among them
#pragma unroll
        for (int q = 0; q < kLgPre; ++q) consume(lgpre[q]);
#pragma unroll
        for (int q = 0; q < kXPre; ++q) consume(xpre[q]);
        lds_barrier();
        const bool pub = blockIdx.x == 0;
        RouteGlobal g{};
        if (pub) g = RouteGlobal{p.ids, p.wts, p.gate_s, const_cast<int *>(p.records),
                                 const_cast<int *>(p.n_unique), const_cast<int *>(p.pairs), p.pos_expert,
                                 p.dbg_ids, p.dbg_w, p.dbg_logits, p.dbg_gate};
        recs = reinterpret_cast<const int *>(area + L.slots);  // 4-int bucket slots
        prs = reinterpret_cast<const int *>(area + L.pairs);
        // Buckets are numbered in order of first appearance, so buckets 0..k-1 are token
        // 0's picks in rank order.  The workgroup's first routed job (bucket `need`, one of
        // those) issues its weight loads as soon as wave 0 has ranked that pick; the rest of
        // the routing (the other picks and tokens, weights, bucketing and tables) runs while
        // the loads are in flight, and the job learns its tokens from the finished buckets.
        // One token needs no bucketing: its k picks are k buckets of one pair each.
        const int fs = j - p.tiles_shared;
        const int need = (!loaded && fs >= 0 && fs / p.tiles_routed < k) ? fs / p.tiles_routed : -1;
        int *lids = reinterpret_cast<int *>(area + L.ids);
        int *lprs = reinterpret_cast<int *>(area + L.pairs);
        int *lpose = reinterpret_cast<int *>(area + L.pose);
        int4 *lslots = reinterpret_cast<int4 *>(area + L.slots);
        float *lw = reinterpret_cast<float *>(area + L.w);
        float *lg1 = reinterpret_cast<float *>(area + L.g);
        int early_e = -1;
        auto route = [&](auto epl) {
            TokenRank<decltype(epl)::value> st;
            // wave 0 lanes r0..r1-1 hold token 0's picks r0..r1-1: their buckets (final for
            // one token; for more tokens only the expert is read before the bucketing
            // rewrites the slots)
            auto publish = [&](int r0, int r1) {
                if (wave == 0 && lane >= r0 && lane < r1) {
                    const int e = (int)st.my_id;
                    lslots[lane] = make_int4(e, lane, 1, 0);
                    lprs[lane] = lane;
                    lpose[lane] = e;
                }
            };
            if (wave == 0) {
                st.begin(lgt, p.E, lane);
                st.rounds(0, need + 1, lane);
            }
            publish(0, need + 1);
            lds_barrier();
            nu = k;
            // a first job of the shared expert issues its loads here too, not before the
            // routing: with one load site for the first job the compiler keeps one register
            // set for it, where two sites made it copy the set at their merge and so wait
            // for the loads in flight there, before the rest of the routing
            if (need >= 0 || j < p.tiles_shared) {
                ja = decode(j);
                if (need >= 0) early_e = lslots[need].x;
                load_rows<WK, LPR, NC, RPW, true>(ja, wave, seg, sl, ag, au, asg, asu, p.swg, p.ssg);
                loaded = true;
            }
            if (wave == 0) {
                st.rounds(need + 1, k, lane);
                publish(need + 1, k);
                // outputs to LDS only (a store that may go to LDS or memory is a flat store,
                // and waiting for one would wait for the weight loads in flight)
                const RouteOut o{lids, lw, lg1, g.dbg_ids, g.dbg_w, g.dbg_gate, g.dbg_logits};
                st.finish(lgt, p.E, k, lane, o);
                if (T == 1 && pub && lane < k) {
                    // the tables the later launches read: bucket `lane` holds pair `lane`
                    const int e = (int)st.my_id;
                    int4 *rec = reinterpret_cast<int4 *>(g.records + lane * kRecInts);
                    rec[0] = make_int4(e, lane, 1, 0);
                    rec[1] = make_int4(lane, -1, -1, -1);
                    rec[2] = make_int4(-1, -1, -1, -1);
                    rec[3] = make_int4(-1, -1, -1, -1);
                    g.ids[lane] = e;
                    g.wts[lane] = lw[lane];  // this lane's own store above
                    g.pairs[lane] = lane;
                    g.pos_expert[lane] = e;
                    if (lane == 0) {
                        *g.n_unique = k;
                        g.gate_s[0] = lg1[0];
                    }
                }
            }
        };
        if (p.E <= 256) route(std::integral_constant<int, 4>{});
        else route(std::integral_constant<int, 8>{});
        if (T == 1) {
            lds_barrier();
        } else {
            // the other tokens (wave w takes tokens w, w + 4, ...; token 0 is done), then the
            // bucketing, whose first barrier orders every wave's picks
            rank_tokens(lgt, 1, T, p.E, k, area, L, g);
            nu = bucket_tokens<SMALL>(T, k, p.E, area, L, g);
            if (need >= 0) {
                // the job's tokens: its bucket as finished (the same expert)
                const int4 sv = lslots[need];
                ja.ntok = sv.z;
                ja.valid = ja.valid && need < nu && sv.x == early_e && sv.y >= 0 && sv.z > 0 &&
                           sv.y + sv.z <= T * k;
            }
        }
        nu = nu < 0 ? 0 : nu > p.E ? p.E : nu;
    }
    const int J = p.tiles_shared + nu * p.tiles_routed;
    if (j >= J) return;
    if (!loaded) {
        ja = decode(j);
        load_rows<WK, LPR, NC, RPW, true>(ja, wave, seg, sl, ag, au, asg, asu, p.swg, p.ssg);
    }
    // tokens staged once (the stage holds the batch; with routing here that is done
    // above) or per pass inside each job; the barrier orders LDS only, so the first job's
    // weight loads stay in flight across it
    if (p.x_resident && !route_here) {
#pragma unroll
        for (int q = 0; q < kXPre; ++q) stage_store(tid + 256 * q, xpre[q], tid + 256 * q < n16);
        lds_barrier();
    }

    // one job's tokens; RES: the stage holds the whole batch (no memory access or barrier
    // in here, so the next job's loads stay in flight while this job computes), else
    // the job's tokens are staged pass by pass
    auto run = [&](auto res, const Job job, const uint4 (&wg)[RPW][NC], const uint4 (&wu)[RPW][NC],
                   const float (&sg)[RPW][NC], const float (&su)[RPW][NC]) {
        constexpr bool RES = decltype(res)::value;
        if (!job.valid) return;
        float *hout = reinterpret_cast<float *>(job.routed ? (uintptr_t)p.h : (uintptr_t)p.hs);
        const int hstride = job.routed ? p.I : p.Is;
        const int tpp = RES ? job.ntok : p.tok_per_pass;
        for (int t0 = 0; t0 < job.ntok; t0 += tpp) {
            const int nt = min(tpp, job.ntok - t0);
            if constexpr (!RES) {
                __syncthreads();
                // rounds of 4 chunks per thread (all loads of a round in flight together)
                const int xr16 = (int)(xrow / 16), n16p = nt * xr16;
                for (int b = 0; b < n16p; b += 1024) {
                uint4 xv[4];
                load_chunks<4>(xv, n16p - b, tid, [&](int ii) {
                    const int i = b + ii;
                    const int a = i / xr16, c = i - a * xr16;
                    int tok = t0 + a;
                    if (job.routed) {
                        const int pr = job_pair<!RH>(job.rec, prs, t0 + a);
                        tok = (pr >= 0 && pr < npairs) ? pr / k : 0;
                    }
                    return (const uint8_t *)p.x + (size_t)tok * xrow + 16 * (size_t)c;
                });
#pragma unroll
                for (int q = 0; q < 4; ++q) stage_store(b + tid + 256 * q, xv[q], b + tid + 256 * q < n16p);
                }
                __syncthreads();
            }
            for (int a = 0; a < nt; ++a) {
                int orow = t0 + a, tok = t0 + a;
                if (job.routed) {
                    orow = job_pair<!RH>(job.rec, prs, t0 + a);
                    tok = orow / k;
                }
                const bool ook = orow >= 0 && orow < (job.routed ? npairs : T);
                const size_t srow = RES ? (size_t)(ook ? tok : 0) : (size_t)a;
                const uint8_t *xr = lds + srow * xrow;
                float g[RPW], u[RPW];
                gate_up_token<WK, LPR, NC, RPW>(xr, xbias + srow * nblk, n_chunks, sl, wg, wu, sg, su, g, u);
                if constexpr (LPR == 64 && (RPW == 1 || RPW == 2)) {
                    // the wave's gate and up rows summed together (gate rows, then up rows),
                    // then each row's gate sum and up sum brought into one lane
                    constexpr int N = 2 * RPW;
                    float pv[N], rs[1];
#pragma unroll
                    for (int i = 0; i < RPW; ++i) {
                        pv[i] = g[i];
                        pv[RPW + i] = u[i];
                    }
                    seg_sum_rows<N>(pv, rs);
                    // lanes holding gate row i: rows_lane<N>(i); its up row sits 32 lanes above
                    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs[0]), __float_as_uint(rs[0]),
                                                                    false, false);
                    const float gs = __uint_as_float(a[0]), us = __uint_as_float(a[1]);
#pragma unroll
                    for (int i = 0; i < RPW; ++i) {
                        const int r = job.tile * RPWG + wave * RPW + i;
                        if (lane == rows_lane<N>(i) && r < job.rows && ook)
                            hout[(size_t)orow * hstride + r] = silu_f(gs) * us;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < RPW; ++i) {
                        const int r = job.tile * RPWG + (wave * RPW + i) * RPI + seg;
                        const float gs = seg_sum<LPR>(g[i]);
                        const float us = seg_sum<LPR>(u[i]);
                        if (sl == 0 && r < job.rows && ook) hout[(size_t)orow * hstride + r] = silu_f(gs) * us;
                    }
                }
            }
        }
    };

    // two jobs per iteration, registers ping-pong between the A and B sets: the next
    // job's loads go out before the current job computes, and the last job of the
    // workgroup runs in a branch of its own, so on every path the compiler knows how
    // many loads are in flight and a job waits only for its own
    auto loop = [&](auto res) {
        for (;;) {
            const int j2 = j + gridDim.x;
            if (j2 >= J) { run(res, ja, ag, au, asg, asu); break; }
            jb = decode(j2);
            load_rows<WK, LPR, NC, RPW, true>(jb, wave, seg, sl, bg, bu, bsg, bsu, p.swg, p.ssg);
            run(res, ja, ag, au, asg, asu);
            j = j2 + gridDim.x;
            if (j >= J) { run(res, jb, bg, bu, bsg, bsu); break; }
            ja = decode(j);
            load_rows<WK, LPR, NC, RPW, true>(ja, wave, seg, sl, ag, au, asg, asu, p.swg, p.ssg);
            run(res, jb, bg, bu, bsg, bsu);
        }
    };
    if (p.x_resident) loop(std::true_type{});
    else loop(std::false_type{});
}

// ---- down: y = down . h per pair, S = shared down . h_s -----------------------------------
// The activation chunk of a lane: EPC fp32 values per 16-byte weight chunk.
template <int WK, int NC>
struct ActChunks {
    float v[NC][WTraits<WK>::epc];
};

template <int WK, int LPR, int NC>
__device__ __forceinline__ void load_act(const float *a, int n_chunks, int sl, ActChunks<WK, NC> &ac) {
    constexpr int EPC = WTraits<WK>::epc;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = sl + LPR * n;
#pragma unroll
        for (int q = 0; q < EPC; q += 4) {
            const float4 v = c < n_chunks ? *reinterpret_cast<const float4 *>(a + EPC * c + q)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
            ac.v[n][q] = v.x; ac.v[n][q + 1] = v.y; ac.v[n][q + 2] = v.z; ac.v[n][q + 3] = v.w;
        }
    }
}

template <int WK, int LPR, int NC, int RPW>
__device__ __forceinline__ float down_dot(const ActChunks<WK, NC> &ac, float (&asum)[NC], int n_chunks,
                                          int sl, const uint4 (&w)[RPW][NC], const float (&s)[RPW][NC],
                                          int i) {
    float acc = 0.f;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        const int c = sl + LPR * n;
        if (c < n_chunks) {
            if constexpr (WK == W_BF16) {
                acc = dot_bf16_f32(w[i][n], make_float4(ac.v[n][0], ac.v[n][1], ac.v[n][2], ac.v[n][3]),
                                   make_float4(ac.v[n][4], ac.v[n][5], ac.v[n][6], ac.v[n][7]), acc);
            } else if constexpr (WK == W_F32) {
                acc = dot_f32_f32(w[i][n], make_float4(ac.v[n][0], ac.v[n][1], ac.v[n][2], ac.v[n][3]), acc);
            } else {
                acc = fmaf(s[i][n], dot_q4_f32(w[i][n], ac.v[n]) - 8.0f * asum[n], acc);
            }
        }
    }
    return acc;
}

template <int WK, int LPR, int NC>
__global__ __launch_bounds__(256) void k_down(DownParams p) {
    constexpr int RPW = WTraits<WK>::rpw_d;
    constexpr int RPI = 64 / LPR;
    constexpr int RPWG = kWaves * RPW * RPI;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg = lane / LPR, sl = lane % LPR;
    const int H = p.H, T = p.T, k = p.k;
    const int npairs = T * k;
    int nu = p.routed ? *p.n_unique : 0;
    nu = nu < 0 ? 0 : nu > p.E ? p.E : nu;
    const int J = p.tiles_shared + nu * p.tiles_routed;
    int j = blockIdx.x;
    if (j >= J) return;

    auto decode = [&](int jj) {
        return decode_job<WK>(jj, p.tiles_shared, p.tiles_routed, nu, p.records, p.E, npairs, p.wd,
                              nullptr, p.sd, nullptr, H, p.I, p.swd, nullptr, p.ssd, nullptr, H, p.Is, T);
    };
    uint4 aw[RPW][NC], bw[RPW][NC], dummy[RPW][NC];
    float as[RPW][NC], bs[RPW][NC], dsc[RPW][NC];
    Job ja = decode(j), jb{};
    load_rows<WK, LPR, NC, RPW, false>(ja, wave, seg, sl, aw, dummy, as, dsc, p.swd, p.ssd);

    auto run = [&](const Job job, const uint4 (&w)[RPW][NC], const float (&s)[RPW][NC]) {
        if (!job.valid) return;
        const int n_chunks = (int)(row_bytes<WK>(job.K) / 16);
        float *dst = reinterpret_cast<float *>(job.routed ? (uintptr_t)p.y : (uintptr_t)p.S);
        for (int a = 0; a < job.ntok; ++a) {
            int orow = a;  // shared: token a
            if (job.routed) {
                orow = job_pair<true>(job.rec, p.pairs, a);
                if (orow < 0 || orow >= npairs) continue;
            }
            // plain integer selects (a pointer select here becomes a table in scratch)
            const uintptr_t abase = job.routed ? (uintptr_t)p.h : (uintptr_t)p.hs;
            const size_t astride = job.routed ? (size_t)p.I : (size_t)p.Is;
            const float *act = reinterpret_cast<const float *>(abase) + (size_t)orow * astride;
            ActChunks<WK, NC> ac;
            load_act<WK, LPR, NC>(act, n_chunks, sl, ac);
            float asum[NC];
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                asum[n] = 0.f;
                if constexpr (WK == W_Q4) {
#pragma unroll
                    for (int q = 0; q < 32; q += 4)
                        asum[n] += (ac.v[n][q] + ac.v[n][q + 1]) + (ac.v[n][q + 2] + ac.v[n][q + 3]);
                }
            }
            if constexpr (LPR == 64) {  // the wave's rows summed together
                float pv[RPW], rs[rows_regs<RPW>()];
#pragma unroll
                for (int i = 0; i < RPW; ++i) pv[i] = down_dot<WK, LPR, NC, RPW>(ac, asum, n_chunks, sl, w, s, i);
                seg_sum_rows<RPW>(pv, rs);
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int r = job.tile * RPWG + wave * RPW + i;
                    if (lane == rows_lane<RPW>(i) && r < job.rows) dst[(size_t)orow * H + r] = rs[rows_reg<RPW>(i)];
                }
            } else {
                float v[RPW];
#pragma unroll
                for (int i = 0; i < RPW; ++i)
                    v[i] = seg_sum<LPR>(down_dot<WK, LPR, NC, RPW>(ac, asum, n_chunks, sl, w, s, i));
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int r = job.tile * RPWG + (wave * RPW + i) * RPI + seg;
                    if (sl == 0 && r < job.rows) dst[(size_t)orow * H + r] = v[i];
                }
            }
        }
    };
    for (;;) {
        const int j2 = j + gridDim.x;
        if (j2 >= J) { run(ja, aw, as); break; }
        jb = decode(j2);
        load_rows<WK, LPR, NC, RPW, false>(jb, wave, seg, sl, bw, dummy, bs, dsc, p.swd, p.ssd);
        run(ja, aw, as);
        j = j2 + gridDim.x;
        if (j >= J) { run(jb, bw, bs); break; }
        ja = decode(j);
        load_rows<WK, LPR, NC, RPW, false>(ja, wave, seg, sl, aw, dummy, as, dsc, p.swd, p.ssd);
        run(jb, bw, bs);
    }
}

// the block's residual input, decoded to fp32 (exact for bf16)
__device__ __forceinline__ float resid_at(const void *x, int is_bf16, size_t i) {
    return is_bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(x)[i] << 16)
                   : reinterpret_cast<const float *>(x)[i];
}

// ---- down + join: one workgroup per tile of output rows (small batches) ---------------------
constexpr int kDJWaves = 16;

// Rows per lane segment of a unit: 8 rows per tile when a row takes one chunk
// per lane, fewer when it takes several.
template <int LPR, int NC>
constexpr int dj_rpw() {
    return (8 * LPR / 64) / NC > 1 ? (8 * LPR / 64) / NC : 1;
}

// A unit is one (token, slot) pair in bucketed order, or one token of the
// shared expert, over the workgroup's whole row tile; 16 waves take units in
// turn, so at small batches every unit's loads are in flight at once.  y for
// the tile stays in LDS and the join runs in place, with the same dot
// products (down_dot + seg_sum over the same row map) and the same join
// arithmetic as k_down + k_join: the results are bit-identical to them.
template <int WK, int LPR, int NC>
__global__ __launch_bounds__(64 * kDJWaves) void k_down_join(DownJoinParams p) {
    constexpr int RPW = dj_rpw<LPR, NC>();
    constexpr int RPI = 64 / LPR;
    constexpr int RT = RPW * RPI;  // rows of the tile
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, sl = lane % LPR;
    const int H = p.H, T = p.T, k = p.k, E = p.E;
    const int NP = T * k, NU = NP + (p.shared_here ? T : 0);
    const int r0 = blockIdx.x * RT;
    int *s_pairs = reinterpret_cast<int *>(lds);          // [NP]
    int *s_pose = s_pairs + NP;                           // [NP]
    float *s_w = reinterpret_cast<float *>(s_pose + NP);  // [NP]
    float *s_g = s_w + NP;                                // [T]
    float *s_y = s_g + T;                                 // [NP + T][RT]
    for (int i = tid; i < NP; i += blockDim.x) {
        s_pairs[i] = p.pairs[i];
        s_pose[i] = p.pos_expert[i];
        s_w[i] = p.wts[i];
    }
    for (int i = tid; i < T; i += blockDim.x) s_g[i] = p.gate_s[i];
    __syncthreads();

    // a unit's loads: every one issued (a row or chunk that does not exist reads the
    // unit's first chunk, an invalid unit the shared matrix; such values are never
    // used), so that with the next unit's loads in flight the current unit waits only
    // for its own
    struct Unit {
        uint4 w[RPW][NC];
        float sc[RPW][NC];
        ActChunks<WK, NC> ac;
        int slot, nch;
        bool ok;
    };
    auto load_unit = [&](int u, Unit &U) {
        const uint8_t *W;
        const uint16_t *Sc = nullptr;
        const float *act;
        int K;
        U.ok = true;
        if (u < NP) {
            const int e = s_pose[u], pr = s_pairs[u];
            U.ok = e >= 0 && e < E && pr >= 0 && pr < NP;
            const size_t m0 = (size_t)(U.ok ? e : 0) * H;
            W = p.wd + m0 * row_bytes<WK>(p.I);
            if constexpr (WK == W_Q4) Sc = p.sd + m0 * (p.I / 32);
            act = p.h + (size_t)(U.ok ? pr : 0) * p.I;
            K = p.I;
            U.slot = U.ok ? pr : 0;
        } else {
            const int t = u - NP;
            W = p.swd;
            if constexpr (WK == W_Q4) Sc = p.ssd;
            act = p.hs + (size_t)t * p.Is;
            K = p.Is;
            U.slot = NP + t;
        }
        const size_t rb = row_bytes<WK>(K);
        const int nch = (int)(rb / 16), nsb = K / 32;
        U.nch = U.ok ? nch : 0;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = r0 + i * RPI + seg;
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                const int c = sl + LPR * n;
                const bool v = U.ok && r < H && c < nch;
                U.w[i][n] = ld16(W + (v ? (size_t)r * rb + 16 * (size_t)c : 0));
                if constexpr (WK == W_Q4) U.sc[i][n] = f16_to_f32(Sc[v ? (size_t)r * nsb + c : 0]);
            }
        }
        constexpr int EPC = WTraits<WK>::epc;
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const int c = sl + LPR * n;
            const float *a = act + (c < nch ? EPC * c : 0);
#pragma unroll
            for (int q = 0; q < EPC; q += 4) {
                const float4 f = *reinterpret_cast<const float4 *>(a + q);
                U.ac.v[n][q] = f.x; U.ac.v[n][q + 1] = f.y; U.ac.v[n][q + 2] = f.z; U.ac.v[n][q + 3] = f.w;
            }
        }
    };
    auto compute_unit = [&](const Unit &U) {
        float asum[NC];
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            asum[n] = 0.f;
            if constexpr (WK == W_Q4) {
#pragma unroll
                for (int q = 0; q < 32; q += 4)
                    asum[n] += (U.ac.v[n][q] + U.ac.v[n][q + 1]) + (U.ac.v[n][q + 2] + U.ac.v[n][q + 3]);
            }
        }
        if constexpr (LPR == 64) {  // the unit's rows summed together
            float pv[RPW], rs[rows_regs<RPW>()];
#pragma unroll
            for (int i = 0; i < RPW; ++i) pv[i] = down_dot<WK, LPR, NC, RPW>(U.ac, asum, U.nch, sl, U.w, U.sc, i);
            seg_sum_rows<RPW>(pv, rs);
#pragma unroll
            for (int i = 0; i < RPW; ++i)
                if (lane == rows_lane<RPW>(i) && U.ok) s_y[U.slot * RT + i] = rs[rows_reg<RPW>(i)];
        } else {
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const float v = seg_sum<LPR>(down_dot<WK, LPR, NC, RPW>(U.ac, asum, U.nch, sl, U.w, U.sc, i));
                if (sl == 0 && U.ok) s_y[U.slot * RT + i * RPI + seg] = v;
            }
        }
    };
    // units in turn per wave, two register sets ping-ponging where a unit's registers are
    // few; the wave's last unit runs in a branch of its own (no load after it)
    constexpr bool DB = RPW * NC * 4 + WTraits<WK>::epc * NC + (WK == W_Q4 ? RPW * NC : 0) <= 48;
    int u = wave;
    if constexpr (!DB) {
        for (; u < NU; u += kDJWaves) {
            Unit A;
            load_unit(u, A);
            compute_unit(A);
        }
    } else if (u < NU) {
        Unit A, B;
        load_unit(u, A);
        for (;;) {
            const int u2 = u + kDJWaves;
            if (u2 >= NU) { compute_unit(A); break; }
            load_unit(u2, B);
            compute_unit(A);
            u = u2 + kDJWaves;
            if (u >= NU) { compute_unit(B); break; }
            load_unit(u, A);
            compute_unit(B);
        }
    }
    __syncthreads();

    // join for the tile's rows of every token (k_join's arithmetic)
    for (int i = tid; i < T * RT; i += blockDim.x) {
        const int t = i / RT, rr = i - t * RT, r = r0 + rr;
        if (r >= H) continue;
        const float *yt = s_y + (size_t)t * k * RT + rr;
        const float *wt = s_w + (size_t)t * k;
        float routed = wt[0] * yt[0];
        for (int j = 1; j < k; ++j) routed = fmaf(wt[j], yt[(size_t)j * RT], routed);
        const float S = p.shared_here ? s_y[(size_t)(NP + t) * RT + rr] : p.S[(size_t)t * H + r];
        float o = __fadd_rn(routed, __fmul_rn(s_g[t], S));
        if (p.resid) o = __fadd_rn(resid_at(p.resid, p.resid_bf16, (size_t)t * H + r), o);
        p.out[(size_t)t * H + r] = o;
    }
}

// ---- join ---------------------------------------------------------------------------------
// out = sum_j w_j y_j + s * S, four columns a thread (hidden sizes are multiples of 32 and
// every tensor is 16-byte aligned): 16-byte loads and stores, one workgroup per 1024
// columns of a token, every load issued before the first use (one memory round trip, not
// k); per column, the products and sums in slot order, the gate product and the final add
// rounded separately.
__global__ __launch_bounds__(256) void k_join(JoinParams p) {
    const int t = blockIdx.y;
    const int r = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (r >= p.H) return;
    const int k = p.k;
    const float *wt = p.wts + (size_t)t * k;
    const float *yr = p.y + (size_t)t * k * p.H + r;
    float4 yv[kMaxTopK];
    float wv[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        yv[j] = j < k ? *reinterpret_cast<const float4 *>(yr + (size_t)j * p.H) : make_float4(0.f, 0.f, 0.f, 0.f);
        wv[j] = j < k ? wt[j] : 0.f;
    }
    const float4 S = *reinterpret_cast<const float4 *>(p.S + (size_t)t * p.H + r);
    const float gs = p.gate_s[t];
    float4 o;
    float *op = &o.x;
    const float *sp = &S.x;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float routed = wv[0] * (&yv[0].x)[c];
#pragma unroll
        for (int j = 1; j < kMaxTopK; ++j)
            if (j < k) routed = fmaf(wv[j], (&yv[j].x)[c], routed);
        float v = __fadd_rn(routed, __fmul_rn(gs, sp[c]));
        if (p.resid) v = __fadd_rn(resid_at(p.resid, p.resid_bf16, (size_t)t * p.H + r + c), v);
        op[c] = v;
    }
    *reinterpret_cast<float4 *>(p.out + (size_t)t * p.H + r) = o;
}

// ---- launchers ----------------------------------------------------------------------------
#define MOE_ROWMAP_CASES(LAUNCH)                  \
    switch (m.lpr * 100 + m.nc) {                 \
    case 801: LAUNCH(8, 1); break;                \
    case 1601: LAUNCH(16, 1); break;              \
    case 3201: LAUNCH(32, 1); break;              \
    case 6401: LAUNCH(64, 1); break;              \
    case 6402: LAUNCH(64, 2); break;              \
    case 6404: LAUNCH(64, 4); break;              \
    case 6408: LAUNCH(64, 8); break;              \
    case 6416: LAUNCH(64, 16); break;             \
    default: return hipErrorInvalidValue;         \
    }

size_t gate_up_lds_bytes(const GateUpParams &p, int xbytes) {
    const int toks = p.x_resident ? p.T : p.tok_per_pass;
    const size_t stage = stage_bytes(toks, p.H, xbytes, p.x_sums);
    return stage + (p.routed && p.route_here ? route_lds_layout(p.T, p.k, p.E, true).bytes : 0);
}

int gate_up_route_lds_off(const GateUpParams &p, int xbytes) {
    const int toks = p.x_resident ? p.T : p.tok_per_pass;
    return (int)stage_bytes(toks, p.H, xbytes, p.x_sums);
}

hipError_t launch_gate_up(const GateUpParams &p, int wkind, const RowMap &m, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    const size_t lds = gate_up_lds_bytes(p, wkind == W_F32 ? 4 : 2);
    if (lds > kLdsLimit) return hipErrorInvalidValue;
    const bool rh = p.routed && p.route_here;
    if ((gate_up_one_row(wkind, m, p.T, rh) || (rh && p.T == 1 && wkind == W_Q4)) &&
        !one_token_stage_fits(p, wkind, m))
        return hipErrorInvalidValue;  // cannot happen: the row map covers the token row
    if (gate_up_one_row(wkind, m, p.T, rh)) {
#define GU_ONE_ROW(L, N) launch_kernel(k_gate_up<W_BF16, 64, N, true, 1>, dim3(grid), dim3(256), lds, s, p);
        switch (m.nc) {
        case 1: GU_ONE_ROW(64, 1); break;
        case 2: GU_ONE_ROW(64, 2); break;
        case 4: GU_ONE_ROW(64, 4); break;
        case 8: GU_ONE_ROW(64, 8); break;
        case 16: GU_ONE_ROW(64, 16); break;
        default: return hipErrorInvalidValue;
        }
#undef GU_ONE_ROW
        return hipGetLastError();
    }
#define GU_BF16_SMALL(L, N) launch_kernel(k_gate_up<W_BF16, L, N, true, 0, false, true>, dim3(grid), dim3(256), lds, s, p);
    if (rh && p.T > 1 && p.T * p.k <= 64 && wkind == W_BF16) {  // bf16, 2-8 tokens of top-8
        MOE_ROWMAP_CASES(GU_BF16_SMALL)
        return hipGetLastError();
    }
#undef GU_BF16_SMALL
#define GU_Q4_ONE(L, N) launch_kernel(k_gate_up<W_Q4, L, N, true, 0, true>, dim3(grid), dim3(256), lds, s, p);
    if (rh && p.T == 1 && wkind == W_Q4) {  // 4-bit rows, one token routed in the workgroups
        MOE_ROWMAP_CASES(GU_Q4_ONE)
        return hipGetLastError();
    }
#undef GU_Q4_ONE
#define GU_LAUNCH_RH(L, N, RH)                                                                               \
    if (wkind == W_F32) launch_kernel(k_gate_up<W_F32, L, N, RH>, dim3(grid), dim3(256), lds, s, p);         \
    else if (wkind == W_BF16) launch_kernel(k_gate_up<W_BF16, L, N, RH>, dim3(grid), dim3(256), lds, s, p);  \
    else launch_kernel(k_gate_up<W_Q4, L, N, RH>, dim3(grid), dim3(256), lds, s, p);
#define GU_LAUNCH(L, N)              \
    if (rh) { GU_LAUNCH_RH(L, N, true) } \
    else { GU_LAUNCH_RH(L, N, false) }
    MOE_ROWMAP_CASES(GU_LAUNCH)
#undef GU_LAUNCH
#undef GU_LAUNCH_RH
    return hipGetLastError();
}

hipError_t launch_down(const DownParams &p, int wkind, const RowMap &m, int grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
#define D_LAUNCH(L, N)                                                                           \
    if (wkind == W_F32) launch_kernel(k_down<W_F32, L, N>, dim3(grid), dim3(256), 0, s, p); \
    else if (wkind == W_BF16) launch_kernel(k_down<W_BF16, L, N>, dim3(grid), dim3(256), 0, s, p); \
    else launch_kernel(k_down<W_Q4, L, N>, dim3(grid), dim3(256), 0, s, p);
    MOE_ROWMAP_CASES(D_LAUNCH)
#undef D_LAUNCH
    return hipGetLastError();
}

int down_join_rows_per_wg(const RowMap &m) {
    const int rpw = std::max(1, (8 * m.lpr / 64) / m.nc);
    return rpw * (64 / m.lpr);
}

size_t down_join_lds_bytes(int T, int k, const RowMap &m) {
    const size_t np = (size_t)T * k;
    return (3 * np + T) * 4 + (np + T) * (size_t)down_join_rows_per_wg(m) * 4;
}

hipError_t launch_down_join(const DownJoinParams &p, int wkind, const RowMap &m, hipStream_t s) {
    const size_t lds = down_join_lds_bytes(p.T, p.k, m);
    if (lds > kLdsLimit) return hipErrorInvalidValue;
    const int rows = down_join_rows_per_wg(m);
    const int grid = (p.H + rows - 1) / rows;
#define DJ_LAUNCH(L, N)                                                                                    \
    if (wkind == W_F32) launch_kernel(k_down_join<W_F32, L, N>, dim3(grid), dim3(64 * kDJWaves), lds, s, p); \
    else if (wkind == W_BF16) launch_kernel(k_down_join<W_BF16, L, N>, dim3(grid), dim3(64 * kDJWaves), lds, s, p); \
    else launch_kernel(k_down_join<W_Q4, L, N>, dim3(grid), dim3(64 * kDJWaves), lds, s, p);
    MOE_ROWMAP_CASES(DJ_LAUNCH)
#undef DJ_LAUNCH
    return hipGetLastError();
}

hipError_t launch_join(const JoinParams &p, hipStream_t s) {
    const bool aligned = (((uintptr_t)p.y | (uintptr_t)p.S | (uintptr_t)p.out) & 15) == 0;
    if (p.H % 4 != 0 || !aligned) return hipErrorInvalidValue;  // the plan and the forward rule these out
    launch_kernel(k_join, dim3((p.H + 1023) / 1024, p.T), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moeffn

namespace moeffn {

// Resident workgroups per CU of the expert kernels (sizes their grid-stride grids).
int expert_kernel_occupancy(bool gate_up, int wkind, const RowMap &m, size_t lds) {
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
#define OCC_CASE(L, N)                                                                            \
    if (gate_up) {                                                                                \
        if (wkind == W_F32) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gate_up<W_F32, L, N, true>, 256, lds); \
        else if (wkind == W_BF16) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gate_up<W_BF16, L, N, true>, 256, lds); \
        else e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gate_up<W_Q4, L, N, true>, 256, lds); \
    } else {                                                                                      \
        if (wkind == W_F32) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_down<W_F32, L, N>, 256, lds); \
        else if (wkind == W_BF16) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_down<W_BF16, L, N>, 256, lds); \
        else e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_down<W_Q4, L, N>, 256, lds); \
    }
    switch (m.lpr * 100 + m.nc) {
    case 801: OCC_CASE(8, 1); break;
    case 1601: OCC_CASE(16, 1); break;
    case 3201: OCC_CASE(32, 1); break;
    case 6401: OCC_CASE(64, 1); break;
    case 6402: OCC_CASE(64, 2); break;
    case 6404: OCC_CASE(64, 4); break;
    case 6408: OCC_CASE(64, 8); break;
    case 6416: OCC_CASE(64, 16); break;
    default: break;
    }
#undef OCC_CASE
    return e == hipSuccess && n > 0 ? n : 1;
}

// The same for the one-row-per-wave gate/up kernel (bf16, 64-lane rows).
int gate_up_one_row_occupancy(const RowMap &m, size_t lds) {
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (m.nc) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gate_up<W_BF16, 64, 1, true, 1>, 256, lds); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gate_up<W_BF16, 64, 2, true, 1>, 256, lds); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gate_up<W_BF16, 64, 4, true, 1>, 256, lds); break;
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gate_up<W_BF16, 64, 8, true, 1>, 256, lds); break;
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gate_up<W_BF16, 64, 16, true, 1>, 256, lds); break;
    default: break;
    }
    return e == hipSuccess && n > 0 ? n : 1;
}

}  // namespace moeffn

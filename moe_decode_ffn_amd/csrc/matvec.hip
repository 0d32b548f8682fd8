// matvec.hip -- small-batch (mat-vec regime) expert kernels.
//
// k_gate_up: one workgroup = one expert (a used routed expert, or the shared
//   expert) x one tile of its intermediate rows.  The tile's gate and up rows
//   are read once into registers with 16-byte loads (a wave instruction reads
//   1 KiB of a row), then applied to every token routed to that expert: the
//   tokens are staged in LDS, each lane pulls its columns, and per row
//   h = silu(gate . x) * (up . x) is written for the (token, slot) pair.
// k_down: one workgroup = one tile of output rows for every token.  It walks
//   the expert-bucketed (token, slot) positions, reading each position's down
//   rows once and the position's h from LDS, keeps y per (pair, row) in LDS,
//   then forms routed = sum_j w_j y_j in slot order and the join
//   out = routed + s * S with the product and the sum rounded separately.
//   The shared expert's rows are extra positions (fused mode), or computed
//   alone into S (shared-only mode), or S is read back (join mode).
// Storage: fp32, bf16, or 4-bit blocks (32 elements + one fp16 scale per
// block, dequantised in registers).
#include "device.h"
#include "internal.h"
#include "routing.h"

namespace moeffn {

constexpr int kWaves = 4;

template <int WK> struct WTraits;
template <> struct WTraits<W_F32> { static constexpr int epc = 4; static constexpr int rpw_gu = 1; };
template <> struct WTraits<W_BF16> { static constexpr int epc = 8; static constexpr int rpw_gu = 2; };
template <> struct WTraits<W_Q4> { static constexpr int epc = 32; static constexpr int rpw_gu = 4; };

static int rpw_gu_of(int wk) {
    return wk == W_F32 ? WTraits<W_F32>::rpw_gu : wk == W_BF16 ? WTraits<W_BF16>::rpw_gu
                                                              : WTraits<W_Q4>::rpw_gu;
}

int gate_up_rows_per_wg(int wkind, const RowMap &m) { return kWaves * rpw_gu_of(wkind) * (64 / m.lpr); }
int down_rows_per_wg(int wkind, const RowMap &m) { (void)wkind; return kWaves * (64 / m.lpr); }

// ---- chunk dot products against bf16 / fp32 activations -------------------------------

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
__device__ __forceinline__ float dot_bf16_f32(uint4 w, const float *a, float acc) {
    const float4 a0 = *reinterpret_cast<const float4 *>(a);
    const float4 a1 = *reinterpret_cast<const float4 *>(a + 4);
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
__device__ __forceinline__ float dot_q4_f32(uint4 w, const float *a) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = ws[i] & 0x0f0f0f0fu, hi = (ws[i] >> 4) & 0x0f0f0f0fu;
        const float4 a0 = *reinterpret_cast<const float4 *>(a + 8 * i);
        const float4 a1 = *reinterpret_cast<const float4 *>(a + 8 * i + 4);
        acc = fmaf((float)(lo & 0xffu), a0.x, acc);
        acc = fmaf((float)(hi & 0xffu), a0.y, acc);
        acc = fmaf((float)((lo >> 8) & 0xffu), a0.z, acc);
        acc = fmaf((float)((hi >> 8) & 0xffu), a0.w, acc);
        acc = fmaf((float)((lo >> 16) & 0xffu), a1.x, acc);
        acc = fmaf((float)((hi >> 16) & 0xffu), a1.y, acc);
        acc = fmaf((float)(lo >> 24), a1.z, acc);
        acc = fmaf((float)(hi >> 24), a1.w, acc);
    }
    return acc;
}

// ---- gate/up ----------------------------------------------------------------------------
template <int WK, int LPR, int NC>
__global__ __launch_bounds__(256) void k_gate_up(GateUpParams p) {
    constexpr int RPW = WTraits<WK>::rpw_gu;
    constexpr int RPI = 64 / LPR;
    constexpr int RPWG = kWaves * RPW * RPI;
    constexpr int XB = WK == W_F32 ? 4 : 2;  // bytes per activation element
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, sl = lane % LPR;
    const int H = p.H, T = p.T, k = p.k, E = p.E;
    const size_t rb = WK == W_F32 ? (size_t)H * 4 : WK == W_BF16 ? (size_t)H * 2 : (size_t)H / 2;
    const int n_chunks = (int)(rb / 16);
    const int nsb = H / 32;  // 4-bit blocks per row
    const int n_pairs = T * k;

    // which expert and tile
    int b = blockIdx.x;
    const uint8_t *Wg, *Wu;
    const uint16_t *Sg = nullptr, *Su = nullptr;
    int n_rows, tile, ntok, start = 0, hstride;
    float *hout;
    const int *pairs = p.pairs;
    bool routed;
    if (b < p.tiles_shared) {
        routed = false;
        Wg = p.swg; Wu = p.swu; Sg = p.ssg; Su = p.ssu;
        n_rows = p.Is; tile = b; ntok = T; hout = p.hs; hstride = p.Is;
    } else {
        routed = true;
        b -= p.tiles_shared;
        const int slot = b / p.tiles_routed;
        tile = b - slot * p.tiles_routed;
        int4 s;
        if (p.route_here) {
            // rank every token of the batch (one wave per token), bucket in LDS
            uint8_t *ra = lds + (size_t)p.tok_per_pass * H * XB;
            int *r_ids = reinterpret_cast<int *>(ra);
            float *r_w = reinterpret_cast<float *>(r_ids + n_pairs);
            float *r_gate = r_w + n_pairs;
            int *r_pairs = reinterpret_cast<int *>(r_gate + T);
            int *r_pose = r_pairs + n_pairs;
            int *r_nu = r_pose + n_pairs;
            int4 *r_slots = reinterpret_cast<int4 *>(ra + (((size_t)(4 * n_pairs + T + 4) * 4 + 15) & ~(size_t)15));
            uint32_t *scratch = reinterpret_cast<uint32_t *>(r_slots + (E < n_pairs ? E : n_pairs));
            const bool publish = b == 0;  // the first routed workgroup writes the tables
            for (int t = wave; t < T; t += kWaves) {
                RouteOut o{r_ids + t * k, r_w + t * k, r_gate + t,
                           publish && p.dbg_ids ? p.dbg_ids + t * k : nullptr,
                           publish && p.dbg_w ? p.dbg_w + t * k : nullptr,
                           publish && p.dbg_gate ? p.dbg_gate + t : nullptr,
                           publish && p.dbg_logits ? p.dbg_logits + (size_t)t * E : nullptr};
                route_token_any(p.logits + (size_t)t * (E + 1), E, k, lane, o);
            }
            __syncthreads();
            bucket_pairs(r_ids, T, k, E, scratch, r_slots, r_pairs, r_pose, r_nu);
            __syncthreads();
            const int nu = *r_nu;
            if (publish) {
                for (int i = tid; i < n_pairs; i += 256) {
                    p.ids[i] = r_ids[i];
                    p.wts[i] = r_w[i];
                    p.pairs[i] = r_pairs[i];
                    p.pos_expert[i] = r_pose[i];
                }
                for (int i = tid; i < T; i += 256) p.gate_s[i] = r_gate[i];
                for (int i = tid; i < nu; i += 256) p.slots[i] = r_slots[i];
                if (tid == 0) *p.n_unique = nu;
            }
            if (slot >= nu) return;
            s = r_slots[slot];
            pairs = r_pairs;
        } else {
            if (slot >= *p.n_unique) return;
            s = p.slots[slot];
        }
        const int e = s.x;
        start = s.y;
        ntok = s.z;
        if (e < 0 || e >= E || start < 0 || ntok <= 0 || start + ntok > n_pairs) return;
        const size_t r0 = (size_t)e * p.I;
        Wg = p.wg + r0 * rb;
        Wu = p.wu + r0 * rb;
        if constexpr (WK == W_Q4) { Sg = p.sg + r0 * nsb; Su = p.su + r0 * nsb; }
        n_rows = p.I; hout = p.h; hstride = p.I;
    }

    int rr[RPW];
    bool rv[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        rr[i] = tile * RPWG + (wave * RPW + i) * RPI + seg;
        rv[i] = rr[i] < n_rows;
    }
    uint4 wg[RPW][NC], wu[RPW][NC];
    float scg[RPW][NC], scu[RPW][NC];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const int c = sl + LPR * n;
            const bool ok = rv[i] && c < n_chunks;
            wg[i][n] = ok ? ld16(Wg + rr[i] * rb + 16 * (size_t)c) : make_uint4(0, 0, 0, 0);
            wu[i][n] = ok ? ld16(Wu + rr[i] * rb + 16 * (size_t)c) : make_uint4(0, 0, 0, 0);
            if constexpr (WK == W_Q4) {
                scg[i][n] = ok ? f16_to_f32(Sg[(size_t)rr[i] * nsb + c]) : 0.f;
                scu[i][n] = ok ? f16_to_f32(Su[(size_t)rr[i] * nsb + c]) : 0.f;
            }
        }

    const int xrow16 = H * XB / 16;
    for (int t0 = 0; t0 < ntok; t0 += p.tok_per_pass) {
        const int nt = min(p.tok_per_pass, ntok - t0);
        __syncthreads();
        for (int i = tid; i < nt * xrow16; i += 256) {
            const int a = i / xrow16, c = i - a * xrow16;
            int tok = t0 + a;
            if (routed) {
                const int pr = pairs[start + t0 + a];
                tok = (pr >= 0 && pr < n_pairs) ? pr / k : 0;
            }
            reinterpret_cast<uint4 *>(lds)[i] =
                ld16((const uint8_t *)p.x + ((size_t)tok * xrow16 + c) * 16);
        }
        __syncthreads();
        for (int a = 0; a < nt; ++a) {
            const uint8_t *xr = lds + (size_t)a * H * XB;
            float g[RPW], u[RPW];
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
                    } else {  // W_Q4: one 32-element block per chunk
                        uint32_t xw[16], xp[16];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint4 v = *reinterpret_cast<const uint4 *>(xr + 64 * c + 16 * q);
                            xw[4 * q + 0] = v.x; xw[4 * q + 1] = v.y;
                            xw[4 * q + 2] = v.z; xw[4 * q + 3] = v.w;
                        }
                        float xsum = 0.f;
#pragma unroll
                        for (int q = 0; q < 16; ++q) xsum += bf16_lo(xw[q]) + bf16_hi(xw[q]);
#pragma unroll
                        for (int q = 0; q < 4; ++q) bf16x8_to_q4_order(xw + 4 * q, xp + 4 * q);
                        const float bias = 136.0f * xsum;  // (128 + 8) * sum x
#pragma unroll
                        for (int i = 0; i < RPW; ++i) {
                            g[i] = fmaf(scg[i][n], dot_q4_bf16(wg[i][n], xp) - bias, g[i]);
                            u[i] = fmaf(scu[i][n], dot_q4_bf16(wu[i][n], xp) - bias, u[i]);
                        }
                    }
                }
            }
            const int orow = routed ? pairs[start + t0 + a] : t0 + a;
            const bool ook = orow >= 0 && orow < (routed ? n_pairs : T);
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const float gs = seg_sum<LPR>(g[i]);
                const float us = seg_sum<LPR>(u[i]);
                if (sl == 0 && rv[i] && ook) hout[(size_t)orow * hstride + rr[i]] = silu_f(gs) * us;
            }
        }
    }
}

// ---- down + weighted sum + join -----------------------------------------------------------
// LDS: act[PP][Kmax] | ybuf[n_pos][RPWG] | pair id and expert per routed position |
//      weights [T*k] | gate [T] | S [T][RPWG] (join mode)
template <int WK, int LPR, int NC>
__global__ __launch_bounds__(256) void k_down(DownParams p) {
    constexpr int RPI = 64 / LPR;
    constexpr int RPWG = kWaves * RPI;
    constexpr int EPC = WTraits<WK>::epc;
    constexpr int QB = NC >= 16 ? 1 : 16 / NC;  // positions whose rows are in registers at once
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, sl = lane % LPR;
    const int H = p.H, k = p.k, T = p.T;
    const int Kmax = p.I > p.Is ? p.I : p.Is;
    const int PP = p.pos_per_pass;                     // <= QB, set by the launcher
    const int n_pos = p.n_routed + p.n_shared;
    const int NPR = T * k;
    float *act = reinterpret_cast<float *>(lds);       // [PP][Kmax]
    float *ybuf = act + (size_t)PP * Kmax;             // [n_pos][RPWG]
    int *t_pair = reinterpret_cast<int *>(ybuf + (size_t)n_pos * RPWG);  // [n_routed]
    int *t_exp = t_pair + p.n_routed;                  // [n_routed]
    float *t_w = reinterpret_cast<float *>(t_exp + p.n_routed);  // [T*k]
    float *t_g = t_w + NPR;                            // [T]
    float *t_S = t_g + T;                              // [T][RPWG]
    const int row0 = blockIdx.x * RPWG;
    const int r = row0 + wave * RPI + seg;
    const bool rv = r < H;
    const int rl = r - row0;

    // tables of this launch, all loads in flight together
    for (int i = tid; i < p.n_routed; i += 256) {
        const int pr = p.pairs[i], e = p.pos_expert[i];
        t_pair[i] = (pr >= 0 && pr < NPR) ? pr : 0;
        t_exp[i] = (e >= 0 && e < p.E) ? e : -1;
    }
    if (p.mode != DOWN_SHARED_ONLY) {
        for (int i = tid; i < NPR; i += 256) t_w[i] = p.wts[i];
        for (int i = tid; i < T; i += 256) t_g[i] = p.gate_s[i];
        if (p.mode == DOWN_JOIN)
            for (int i = tid; i < T * RPWG; i += 256) {
                const int t = i / RPWG, c = i - t * RPWG;
                t_S[i] = row0 + c < H ? p.S_in[(size_t)t * H + row0 + c] : 0.f;
            }
    }
    __syncthreads();

    for (int q0 = 0; q0 < n_pos; q0 += PP) {
        const int nq = min(PP, n_pos - q0);
        uint4 w[QB][NC];
        float sc[QB][NC];
        int nch[QB];
#pragma unroll
        for (int a = 0; a < QB; ++a) {
            const int q = q0 + a;
            const uint8_t *Wm = p.swd;
            const uint16_t *Sm = p.ssd;
            int K = p.Is;
            bool ok = a < nq;
            if (ok && q < p.n_routed) {
                const int e = t_exp[q];
                ok = e >= 0;
                K = p.I;
                const size_t rbk = WK == W_F32 ? (size_t)K * 4 : WK == W_BF16 ? (size_t)K * 2 : (size_t)K / 2;
                Wm = p.wd + (size_t)(ok ? e : 0) * H * rbk;
                if constexpr (WK == W_Q4) Sm = p.sd + (size_t)(ok ? e : 0) * H * (K / 32);
            }
            const size_t rbk = WK == W_F32 ? (size_t)K * 4 : WK == W_BF16 ? (size_t)K * 2 : (size_t)K / 2;
            nch[a] = (int)(rbk / 16);
#pragma unroll
            for (int n = 0; n < NC; ++n) {
                const int c = sl + LPR * n;
                const bool okc = ok && rv && c < nch[a];
                w[a][n] = okc ? ld16(Wm + (size_t)r * rbk + 16 * (size_t)c) : make_uint4(0, 0, 0, 0);
                if constexpr (WK == W_Q4)
                    sc[a][n] = okc ? f16_to_f32(Sm[(size_t)r * (K / 32) + c]) : 0.f;
            }
        }
        if (q0 > 0) __syncthreads();  // the previous pass is done with act[]
        const int k4 = Kmax / 4;
        for (int i = tid; i < nq * k4; i += 256) {
            const int a = i / k4, c4 = i - a * k4;
            const int q = q0 + a;
            const float *src;
            int K;
            if (q < p.n_routed) {
                src = p.h + (size_t)t_pair[q] * p.I;
                K = p.I;
            } else {
                src = p.hs + (size_t)(q - p.n_routed) * p.Is;
                K = p.Is;
            }
            if (4 * c4 < K)
                reinterpret_cast<float4 *>(act)[i] = *reinterpret_cast<const float4 *>(src + 4 * c4);
        }
        __syncthreads();
#pragma unroll
        for (int a = 0; a < QB; ++a) {
            if (a < nq) {
                const float *av = act + (size_t)a * Kmax;
                float acc = 0.f;
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    const int c = sl + LPR * n;
                    if (c < nch[a]) {
                        if constexpr (WK == W_BF16) {
                            acc = dot_bf16_f32(w[a][n], av + EPC * c, acc);
                        } else if constexpr (WK == W_F32) {
                            acc = dot_f32_f32(w[a][n], *reinterpret_cast<const float4 *>(av + EPC * c), acc);
                        } else {
                            const float *ab = av + EPC * c;
                            float asum = 0.f;
#pragma unroll
                            for (int q = 0; q < 32; q += 4) {
                                const float4 v = *reinterpret_cast<const float4 *>(ab + q);
                                asum += (v.x + v.y) + (v.z + v.w);
                            }
                            acc = fmaf(sc[a][n], dot_q4_f32(w[a][n], ab) - 8.0f * asum, acc);
                        }
                    }
                }
                acc = seg_sum<LPR>(acc);
                const int q = q0 + a;
                const int slot = q < p.n_routed ? t_pair[q] : q;
                if (sl == 0 && rv) ybuf[(size_t)slot * RPWG + rl] = acc;
            }
        }
    }
    __syncthreads();

    for (int i = tid; i < T * RPWG; i += 256) {
        const int t = i / RPWG, c = i - t * RPWG;
        const int rr = row0 + c;
        if (rr >= H) continue;
        if (p.mode == DOWN_SHARED_ONLY) {
            p.S_out[(size_t)t * H + rr] = ybuf[(size_t)t * RPWG + c];
            continue;
        }
        const float *wt = t_w + (size_t)t * k;
        const float *yr = ybuf + (size_t)t * k * RPWG + c;
        float routed = wt[0] * yr[0];
        for (int j = 1; j < k; ++j) routed = fmaf(wt[j], yr[(size_t)j * RPWG], routed);
        const float S = p.mode == DOWN_FUSED ? ybuf[(size_t)(p.n_routed + t) * RPWG + c] : t_S[i];
        p.out[(size_t)t * H + rr] = __fadd_rn(routed, __fmul_rn(t_g[t], S));
    }
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

hipError_t launch_gate_up(const GateUpParams &p, int wkind, const RowMap &m, int rows_per_wg,
                          int grid, size_t lds, hipStream_t s) {
    (void)rows_per_wg;
    if (grid <= 0) return hipSuccess;
    lds = gate_up_lds_bytes(p, wkind == W_F32 ? 4 : 2);
    if (lds > kLdsLimit) return hipErrorInvalidValue;
#define GU_LAUNCH(L, N)                                                                          \
    if (wkind == W_F32) hipLaunchKernelGGL((k_gate_up<W_F32, L, N>), dim3(grid), dim3(256), lds, s, p); \
    else if (wkind == W_BF16) hipLaunchKernelGGL((k_gate_up<W_BF16, L, N>), dim3(grid), dim3(256), lds, s, p); \
    else hipLaunchKernelGGL((k_gate_up<W_Q4, L, N>), dim3(grid), dim3(256), lds, s, p);
    MOE_ROWMAP_CASES(GU_LAUNCH)
#undef GU_LAUNCH
    return hipGetLastError();
}

size_t down_lds_bytes(int wkind, const RowMap &m, int I, int Is, int T, int k, int n_routed,
                      int n_shared, int *pos_per_pass) {
    const int qb = m.nc >= 16 ? 1 : 16 / m.nc;
    const int Kmax = I > Is ? I : Is;
    int pp = (int)(kStageBytes / ((size_t)Kmax * 4));
    pp = pp < 1 ? 1 : pp > qb ? qb : pp;
    const int rpwg = down_rows_per_wg(wkind, m);
    const size_t fixed = (size_t)(n_routed + n_shared) * rpwg + 2 * (size_t)n_routed + (size_t)T * k + T +
                         (size_t)T * rpwg;
    while (pp > 1 && (fixed + (size_t)pp * Kmax) * 4 > kLdsLimit) pp >>= 1;  // fewer staged vectors
    if (pos_per_pass) *pos_per_pass = pp;
    return (fixed + (size_t)pp * Kmax) * 4;
}

size_t gate_up_lds_bytes(const GateUpParams &p, int xbytes) {
    size_t b = (size_t)p.tok_per_pass * p.H * xbytes;
    if (p.route_here) {
        const int np = p.T * p.k;
        b += (((size_t)(4 * np + p.T + 4) * 4 + 15) & ~(size_t)15) + (size_t)(p.E < np ? p.E : np) * 16 +
             (size_t)bucket_scratch_ints(p.E, p.T) * 4;
    }
    return b;
}

hipError_t launch_down(const DownParams &p_in, int wkind, const RowMap &m, int rows_per_wg,
                       int grid, size_t lds, hipStream_t s) {
    (void)rows_per_wg;
    if (grid <= 0) return hipSuccess;
    DownParams p = p_in;
    lds = down_lds_bytes(wkind, m, p.I, p.Is, p.T, p.k, p.n_routed, p.n_shared, &p.pos_per_pass);
    if (lds > kLdsLimit) return hipErrorInvalidValue;
#define D_LAUNCH(L, N)                                                                           \
    if (wkind == W_F32) hipLaunchKernelGGL((k_down<W_F32, L, N>), dim3(grid), dim3(256), lds, s, p); \
    else if (wkind == W_BF16) hipLaunchKernelGGL((k_down<W_BF16, L, N>), dim3(grid), dim3(256), lds, s, p); \
    else hipLaunchKernelGGL((k_down<W_Q4, L, N>), dim3(grid), dim3(256), lds, s, p);
    MOE_ROWMAP_CASES(D_LAUNCH)
#undef D_LAUNCH
    return hipGetLastError();
}

}  // namespace moeffn

// forward.cpp -- moe_ffn_forward / moe_ffn_destroy / profiling hooks.
//
// Kernels of one forward:
//   router  logits of E router rows and of the shared-gate vector
//   routing top-k, renormalised weights, bucketing, job records: in every
//           routed mat-vec gate/up workgroup (up to 16 tokens, when the batch's
//           logits rows and routing tables fit that launch's LDS), else in a
//           routing launch of its own (k_route, one workgroup, up to 16 tokens),
//           else in three batch launches (ranking with per-workgroup expert
//           counts, a per-expert scan of the counts, the placement of the pairs)
//   gate/up h = silu(gate x) * (up x) for every (token, slot) pair [+ shared]
//   down    y = down h per pair [+ S for the shared expert]
//   join    out = sum_j w_j y_j + s * S (mat-vec regime: k_down_join does the
//           down step and the join in one launch)
// gate/up and down are mat-vec kernels (matvec.hip) up to matvec_max tokens and
// grouped MFMA GEMMs (gemm.hip) above it when the storage is bf16.
// Where the shared expert's gate/up and down run (page "ggml-cuda: overlap the
// MoE shared expert on a separate stream", section "What this changes": one
// fork at the input, one join before the add):
//   AUX   on the plan's second stream, forked from `stream` at entry and joined
//         by an event just before the join kernel
//   SEQ   the same kernels on `stream`, before the routed chain
//   FUSED as extra jobs of the routed gate/up and down launches
// Every mode runs the same per-element arithmetic, so their outputs are
// bit-identical (the pages' requirement that the overlapped output equal the
// sequential one).
#include <algorithm>
#include <cstring>
#include <string>

#include "internal.h"

using namespace moeffn;

namespace moeffn {
thread_local LaunchEvents g_launch_events;
}

namespace {

struct Range {
    const void *p;
    size_t n;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_ffn_status hip_fail(hipError_t e, const char *what) {
    return set_error(MOE_FFN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

hipEvent_t pool_event(moe_ffn_plan_s *P) {
    if (!P->pool.empty()) {
        hipEvent_t e = P->pool.back();
        P->pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Runs `launch` on stream s; when profiling, the kernel's own dispatch records
// a pair of timing events (its start and end), so the interval is the
// kernel's duration without the gaps around it.
template <class F>
hipError_t timed(moe_ffn_plan_s *P, int kernel, hipStream_t s, F &&launch) {
    if (!P->profiling) return launch();
    hipEvent_t a = pool_event(P), b = pool_event(P);
    if (!a || !b) return hipErrorOutOfMemory;
    g_launch_events = LaunchEvents{a, b};
    hipError_t e = launch();
    if (g_launch_events.start) {  // nothing was launched (an empty grid): a zero interval
        g_launch_events = LaunchEvents{};
        if (e == hipSuccess) e = hipEventRecord(a, s);
        if (e == hipSuccess) e = hipEventRecord(b, s);
    }
    if (e != hipSuccess) return e;
    P->prof.push_back({kernel, a, b});
    return e;
}

moe_ffn_status lazy_init(moe_ffn_plan_s *P, hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
        return set_error(MOE_FFN_ERR_UNSUPPORTED,
                         "the first forward of a plan creates its stream and events and must not be captured");
    // the second stream and its events exist only for a plan that forks onto it
    if (P->mode_matvec == MOE_FFN_SHARED_AUX || P->mode_gemm == MOE_FFN_SHARED_AUX) {
        if ((e = hipStreamCreateWithFlags(&P->aux, hipStreamNonBlocking)) != hipSuccess)
            return hip_fail(e, "hipStreamCreateWithFlags");
        if ((e = hipEventCreateWithFlags(&P->ev_fork, hipEventDisableTiming)) != hipSuccess)
            return hip_fail(e, "hipEventCreateWithFlags");
        if ((e = hipEventCreateWithFlags(&P->ev_join, hipEventDisableTiming)) != hipSuccess)
            return hip_fail(e, "hipEventCreateWithFlags");
    }
    if ((e = hipDeviceGetAttribute(&P->cu_count, hipDeviceAttributeMultiprocessorCount, P->d.device)) != hipSuccess)
        return hip_fail(e, "hipDeviceGetAttribute");
    P->occ_gu = expert_kernel_occupancy(true, P->wkind, P->map_gu, kStageBytes);
    P->occ_gu1 = P->map_gu.lpr == 64 ? gate_up_one_row_occupancy(P->map_gu, kStageBytes) : 1;
    P->occ_d = expert_kernel_occupancy(false, P->wkind, P->map_down, 0);
    if (P->gemm_ok) {
        for (int i = 0; i < 3; ++i) {
            P->occ_gg_gu[i] = gg_occupancy(true, 1 << i);
            P->occ_gg_d[i] = gg_occupancy(false, 1 << i);
        }
        for (int i = 0; i < 3; ++i) {
            P->occ_pf_gu[i] = pf_occupancy(true, 2 + i);
            P->occ_pf_d[i] = pf_occupancy(false, 2 + i);
        }
    }
    P->ready = true;
    return MOE_FFN_OK;
}

}  // namespace

extern "C" {

moe_ffn_status moe_ffn_forward(moe_ffn_plan_t P, const moe_ffn_tensors *t, int32_t n_tokens,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!P || !t) return set_error(MOE_FFN_ERR_INVALID_ARG, "plan and tensors must not be NULL");
    const moe_ffn_desc &d = P->d;
    if (n_tokens < 0 || n_tokens > d.max_tokens)
        return set_error(MOE_FFN_ERR_TOO_MANY_TOKENS, "n_tokens must be in [0, max_tokens]");
    if (n_tokens == 0) return MOE_FFN_OK;

    const bool q4 = d.weight_dtype == MOE_FFN_Q4_B32;
    const void *req[] = {t->x, t->w_router, t->w_gate, t->w_up, t->w_down, t->sh_gate,
                         t->sh_up, t->sh_down, t->gate_vec, t->out};
    for (const void *p : req)
        if (!p) return set_error(MOE_FFN_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    const void *sc[] = {t->w_gate_scale, t->w_up_scale, t->w_down_scale, t->sh_gate_scale,
                        t->sh_up_scale, t->sh_down_scale};
    for (const void *p : sc)
        if ((p != nullptr) != q4)
            return set_error(MOE_FFN_ERR_INVALID_ARG, "scale pointers must be set exactly for Q4_B32 storage");
    const bool norm = d.flags & MOE_FFN_INPUT_NORM;
    if ((t->norm_weight != nullptr) != norm)
        return set_error(MOE_FFN_ERR_INVALID_ARG, "norm_weight must be set exactly when INPUT_NORM is");
    if (!workspace) return set_error(MOE_FFN_ERR_INVALID_ARG, "workspace must not be NULL");
    if (workspace_bytes < P->L.total)
        return set_error(MOE_FFN_ERR_WORKSPACE_TOO_SMALL,
                         "workspace needs " + std::to_string(P->L.total) + " bytes");
    if (!aligned(workspace, kWsAlign)) return set_error(MOE_FFN_ERR_MISALIGNED, "workspace not 256-byte aligned");
    const void *all[] = {t->x, t->w_router, t->w_gate, t->w_up, t->w_down, t->w_gate_scale,
                         t->w_up_scale, t->w_down_scale, t->sh_gate, t->sh_up, t->sh_down,
                         t->sh_gate_scale, t->sh_up_scale, t->sh_down_scale, t->gate_vec, t->out,
                         t->dbg_topk_ids, t->dbg_topk_weights, t->dbg_logits, t->dbg_shared_gate,
                         t->norm_weight};
    for (const void *p : all)
        if (!aligned(p, 16)) return set_error(MOE_FFN_ERR_MISALIGNED, "tensor pointers must be 16-byte aligned");

    // aliasing: out may equal x exactly (same bytes, fp32 x), nothing else may overlap it
    const size_t T = (size_t)n_tokens, H = d.hidden, E = d.n_experts, k = d.top_k;
    const size_t I = d.inter, Is = d.shared_inter;
    const size_t xb = d.x_dtype == MOE_FFN_F32 ? 4 : 2;
    const int wk = P->wkind;
    const Range out{t->out, T * H * 4};
    const Range ins[] = {
        {t->w_router, E * H * 4},
        {t->w_gate, E * I * row_bytes_of(wk, (int)H)},
        {t->w_up, E * I * row_bytes_of(wk, (int)H)},
        {t->w_down, E * H * row_bytes_of(wk, (int)I)},
        {t->w_gate_scale, q4 ? E * I * (H / 32) * 2 : 0},
        {t->w_up_scale, q4 ? E * I * (H / 32) * 2 : 0},
        {t->w_down_scale, q4 ? E * H * (I / 32) * 2 : 0},
        {t->sh_gate, Is * row_bytes_of(wk, (int)H)},
        {t->sh_up, Is * row_bytes_of(wk, (int)H)},
        {t->sh_down, H * row_bytes_of(wk, (int)Is)},
        {t->sh_gate_scale, q4 ? Is * (H / 32) * 2 : 0},
        {t->sh_up_scale, q4 ? Is * (H / 32) * 2 : 0},
        {t->sh_down_scale, q4 ? H * (Is / 32) * 2 : 0},
        {t->gate_vec, H * 4},
        {t->norm_weight, norm ? H * 4 : 0},
        {workspace, P->L.total},
        {t->dbg_topk_ids, t->dbg_topk_ids ? T * k * 4 : 0},
        {t->dbg_topk_weights, t->dbg_topk_weights ? T * k * 4 : 0},
        {t->dbg_logits, t->dbg_logits ? T * E * 4 : 0},
        {t->dbg_shared_gate, t->dbg_shared_gate ? T * 4 : 0},
    };
    for (const Range &r : ins)
        if (overlap(out, r)) return set_error(MOE_FFN_ERR_ALIAS, "out overlaps an input, the workspace or a debug output");
    const Range xr{t->x, T * H * xb};
    if (overlap(out, xr) && !(t->out == t->x && xb == 4))
        return set_error(MOE_FFN_ERR_ALIAS, "out may alias x only exactly (fp32 x)");
    const Range ws{workspace, P->L.total};
    if (overlap(xr, ws)) return set_error(MOE_FFN_ERR_ALIAS, "x overlaps the workspace");

    // device checks
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != d.device) return set_error(MOE_FFN_ERR_WRONG_DEVICE, "current device differs from desc.device");
    if (stream) {
        hipDevice_t sd = -1;
        if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        if (sd != d.device) return set_error(MOE_FFN_ERR_WRONG_DEVICE, "stream belongs to another device");
    }
    if (!P->ready) {
        moe_ffn_status st = lazy_init(P, stream);
        if (st != MOE_FFN_OK) return st;
    }

    // workspace views
    uint8_t *W = (uint8_t *)workspace;
    const Layout &L = P->L;
    float *sh_h = (float *)(W + L.sh_h), *sh_S = (float *)(W + L.sh_S);
    float *gate_s = (float *)(W + L.gate_s), *wts = (float *)(W + L.wts);
    int *ids = (int *)(W + L.ids), *n_unique = (int *)(W + L.n_unique);
    int *pairs = (int *)(W + L.pairs), *pos_expert = (int *)(W + L.pos_expert);
    int *records = (int *)(W + L.records);
    float *logits = (float *)(W + L.logits), *h = (float *)(W + L.h), *y = (float *)(W + L.y);
    // the experts' input: x, or the router's normalised copy of it
    const void *xe = norm ? (const void *)(W + L.xn) : t->x;
    const void *resid = (d.flags & MOE_FFN_RESIDUAL) ? t->x : nullptr;

    const uint32_t mode = n_tokens <= P->matvec_max ? P->mode_matvec : P->mode_gemm;
    const bool gemm = P->gemm_ok && ((d.flags & MOE_FFN_FORCE_GEMM) || n_tokens > P->matvec_max);
    const int Ti = n_tokens;

    RouterParams rp{};
    rp.x = t->x;
    rp.x_bf16 = d.x_dtype == MOE_FFN_BF16;
    rp.T = Ti; rp.H = (int)H; rp.E = (int)E;
    rp.router = t->w_router; rp.gate_vec = t->gate_vec; rp.logits = logits;
    // tokens per router workgroup: up to 8 (the GEMV router serves up to 16 bf16 tokens,
    // and fp32 tokens or the input norm at any batch; one workgroup per row and tile)
    rp.tok_tile = std::max(1, std::min(8, (int)(kStageBytes / (H * xb))));
    const int r_tiles = (Ti + rp.tok_tile - 1) / rp.tok_tile;

    rp.k = (int)k;
    rp.ids = ids; rp.wts = wts; rp.gate_s = gate_s; rp.records = records; rp.n_unique = n_unique;
    rp.pairs = pairs; rp.pos_expert = pos_expert;
    rp.dbg_ids = t->dbg_topk_ids; rp.dbg_w = t->dbg_topk_weights;
    rp.dbg_logits = t->dbg_logits; rp.dbg_gate = t->dbg_shared_gate;
    rp.norm_w = t->norm_weight; rp.norm_eps = d.norm_eps; rp.xn = W + L.xn;

    GateUpParams gp{};
    gp.x = xe; gp.T = Ti; gp.H = (int)H; gp.k = (int)k; gp.E = (int)E;
    gp.x_resident = (size_t)Ti * H * xb <= kStageBytes ? 1 : 0;
    gp.tok_per_pass = std::max(1, (int)(kStageBytes / (H * xb)));
    gp.x_sums = wk == W_Q4 ? 1 : 0;
    gp.wg = (const uint8_t *)t->w_gate; gp.wu = (const uint8_t *)t->w_up;
    gp.sg = t->w_gate_scale; gp.su = t->w_up_scale; gp.I = (int)I;
    gp.records = records; gp.n_unique = n_unique; gp.pairs = pairs; gp.h = h;
    gp.swg = (const uint8_t *)t->sh_gate; gp.swu = (const uint8_t *)t->sh_up;
    gp.ssg = t->sh_gate_scale; gp.ssu = t->sh_up_scale; gp.Is = (int)Is; gp.hs = sh_h;
    // small batches: every routed gate/up workgroup ranks and buckets the batch from
    // the logits (no routing step between the router and the experts); otherwise a
    // routing launch of its own (up to 16 tokens) or the batch routing launches
    gp.logits = logits; gp.ids = ids; gp.wts = wts; gp.gate_s = gate_s; gp.pos_expert = pos_expert;
    gp.dbg_ids = t->dbg_topk_ids; gp.dbg_w = t->dbg_topk_weights;
    gp.dbg_logits = t->dbg_logits; gp.dbg_gate = t->dbg_shared_gate;
    {
        GateUpParams q = gp;
        q.routed = 1;
        q.route_here = 1;
        // (the prologue holds the batch's logits rows in at most 5 chunks per thread)
        gp.route_here = !gemm && Ti <= kRouteInGateUpMax && (size_t)Ti * logit_stride((int)E) / 4 <= 5 * 256 &&
                        gate_up_lds_bytes(q, (int)xb) <= kLdsLimit ? 1 : 0;
        gp.route_lds_off = gate_up_route_lds_off(q, (int)xb);
    }
    // else a routing launch of its own (one wave per token, up to 16 tokens)
    const bool route_kernel = !gp.route_here && Ti <= kRouteKernelMax &&
                              route_kernel_lds_bytes(Ti, (int)k, (int)E) <= kLdsLimit;
    // larger batches (or a shape whose routing does not fit in LDS): ranking and
    // bucketing launches of their own, through global memory
    const bool batch_route = !gp.route_here && !route_kernel;
    rp.bcount = batch_route ? (int *)(W + L.bcount) : nullptr;
    const int max_used = (int)std::min(E, T * k);

    DownParams dp{};
    dp.T = Ti; dp.H = (int)H; dp.k = (int)k; dp.E = (int)E;
    dp.wd = (const uint8_t *)t->w_down; dp.sd = t->w_down_scale; dp.I = (int)I;
    dp.h = h; dp.records = records; dp.n_unique = n_unique; dp.pairs = pairs; dp.y = y;
    dp.swd = (const uint8_t *)t->sh_down; dp.ssd = t->sh_down_scale; dp.Is = (int)Is;
    dp.hs = sh_h; dp.S = sh_S;
    const int d_rows = down_rows_per_wg(wk, P->map_down);
    dp.tiles_routed = (int)((H + d_rows - 1) / d_rows);
    const int d_tiles_s = dp.tiles_routed;

    // grouped-GEMM regime: h is kept in bf16 (the down GEMM's operand) in the same regions
    GGParams gg{};
    gg.x = xe; gg.T = Ti; gg.H = (int)H; gg.k = (int)k; gg.E = (int)E; gg.I = (int)I;
    gg.Is = (int)Is; gg.records = records; gg.n_unique = n_unique; gg.pairs = pairs;
    gg.hb = (uint16_t *)h; gg.shb = (uint16_t *)sh_h; gg.y = y; gg.S = sh_S;
    const int gg_rows = gg_rows_per_job();
    // 16 tokens per MFMA tile; a pass takes 1, 2 or 4 tiles by the mean bucket size (more
    // tokens per pass read each expert's weights fewer times); the shared expert's tokens
    // are split into blocks of one pass
    const size_t mean_bucket = T * k / std::max<size_t>(1, std::min(E, T * k));
    const int gg_nt = mean_bucket >= 48 ? 4 : mean_bucket >= 24 ? 2 : 1;
    // large buckets: the prefill GEMM (weight stages shared through LDS, 128, 192 or 256 tokens
    // per pass)
    const bool pf = gemm && mean_bucket >= (size_t)kPfMinBucket;
    // one pass per bucket where possible: 192 tokens cover buckets up to ~1.5x a mean of 128
    const int pf_ntw = mean_bucket >= 192 ? 4 : mean_bucket >= 96 ? 3 : 2;
    const int gg_tb = (Ti + 16 * gg_nt - 1) / (16 * gg_nt);
    auto nt_index = [](int nt) { return nt <= 1 ? 0 : nt <= 2 ? 1 : 2; };

    // mat-vec regime: down and join in one launch when the row tile's y fits in LDS
    const bool use_dj = !gemm && !(d.flags & MOE_FFN_DEBUG_SPLIT_JOIN) &&
                        down_join_lds_bytes(Ti, (int)k, P->map_down) <= kLdsLimit;
    DownJoinParams djp{};
    djp.T = Ti; djp.H = (int)H; djp.k = (int)k; djp.E = (int)E;
    djp.wd = (const uint8_t *)t->w_down; djp.sd = t->w_down_scale; djp.I = (int)I; djp.h = h;
    djp.pairs = pairs; djp.pos_expert = pos_expert;
    djp.swd = (const uint8_t *)t->sh_down; djp.ssd = t->sh_down_scale; djp.Is = (int)Is; djp.hs = sh_h;
    djp.S = sh_S; djp.wts = wts; djp.gate_s = gate_s; djp.out = t->out;
    djp.resid = resid; djp.resid_bf16 = d.x_dtype == MOE_FFN_BF16;

    JoinParams jp{};
    jp.T = Ti; jp.H = (int)H; jp.k = (int)k; jp.y = y; jp.wts = wts; jp.gate_s = gate_s;
    jp.S = sh_S; jp.out = t->out;
    jp.resid = resid; jp.resid_bf16 = d.x_dtype == MOE_FFN_BF16;

    const bool delay_main = d.flags & MOE_FFN_DEBUG_DELAY_MAIN;
    const bool delay_aux = d.flags & MOE_FFN_DEBUG_DELAY_AUX;
    const uint64_t delay_ticks = 20000;  // 200 us of the 100 MHz constant clock

    // large batches of bf16 tokens without the input norm: the router as an MFMA GEMM
    const bool router_mfma = batch_route && rp.x_bf16 && !norm && H % 128 == 0;
    auto run_router = [&](hipStream_t s) {
        hipError_t e1 = timed(P, MOE_FFN_K_ROUTER, s, [&] {
            return router_mfma ? launch_router_mfma(rp, s) : launch_router(rp, r_tiles, s);
        });
        if (e1 != hipSuccess) return e1;
        if (route_kernel) return timed(P, MOE_FFN_K_ROUTE, s, [&] { return launch_route(rp, s); });
        if (!batch_route) return e1;
        e1 = timed(P, MOE_FFN_K_ROUTE, s, [&] { return launch_rank_batch(rp, s); });
        if (e1 != hipSuccess) return e1;
        e1 = timed(P, MOE_FFN_K_BUCKET, s, [&] { return launch_count_scan(rp, s); });
        if (e1 != hipSuccess) return e1;
        return timed(P, MOE_FFN_K_BUCKET, s, [&] { return launch_bucket_batch(rp, s); });
    };
    // grid of a grid-stride expert launch: its jobs, capped at the resident workgroups
    auto expert_grid = [&](int jobs, int occ) { return std::max(1, std::min(jobs, occ * P->cu_count)); };
    auto run_gate_up = [&](hipStream_t s, bool routed, bool shared) {
        GateUpParams g = gp;
        g.routed = routed ? 1 : 0;
        // rows per job depend on the kernel this launch takes (routing here or not)
        const bool one_row = gate_up_one_row(wk, P->map_gu, Ti, routed && g.route_here);
        const int gu_rows = gate_up_rows_per_wg(wk, P->map_gu, Ti, routed && g.route_here);
        g.tiles_routed = (int)((I + gu_rows - 1) / gu_rows);
        g.tiles_shared = shared ? (int)((Is + gu_rows - 1) / gu_rows) : 0;
        const int jobs = g.tiles_shared + (routed ? max_used * g.tiles_routed : 0);
        const int kid = routed ? MOE_FFN_K_GATE_UP : MOE_FFN_K_SH_GATE_UP;
        return timed(P, kid, s, [&] {
            return launch_gate_up(g, wk, P->map_gu, expert_grid(jobs, one_row ? P->occ_gu1 : P->occ_gu), s);
        });
    };
    auto run_down = [&](hipStream_t s, bool routed, bool shared) {
        DownParams q = dp;
        q.routed = routed ? 1 : 0;
        q.tiles_shared = shared ? d_tiles_s : 0;
        const int jobs = q.tiles_shared + (routed ? max_used * q.tiles_routed : 0);
        const int kid = routed ? MOE_FFN_K_DOWN : MOE_FFN_K_SH_DOWN;
        return timed(P, kid, s, [&] {
            return launch_down(q, wk, P->map_down, expert_grid(jobs, P->occ_d), s);
        });
    };
    auto run_pf = [&](hipStream_t s, bool gate_up, bool routed, bool shared) {
        GGParams g = gg;
        if (gate_up) {
            g.w0 = (const uint8_t *)t->w_gate; g.w1 = (const uint8_t *)t->w_up;
            g.sw0 = (const uint8_t *)t->sh_gate; g.sw1 = (const uint8_t *)t->sh_up;
        } else {
            g.w0 = (const uint8_t *)t->w_down; g.sw0 = (const uint8_t *)t->sh_down;
        }
        const int rows = pf_rows_per_job(gate_up);
        g.routed = routed ? 1 : 0;
        g.tiles_routed = (int)(((gate_up ? I : H) + rows - 1) / rows);
        g.tiles_shared = shared ? (int)(((gate_up ? Is : H) + rows - 1) / rows) : 0;
        const int bn = pf_tokens_per_pass(pf_ntw);
        const int jobs = pf_job_count(g.tiles_shared, (Ti + bn - 1) / bn, routed ? max_used : 0, g.tiles_routed);
        const int occ = (gate_up ? P->occ_pf_gu : P->occ_pf_d)[pf_ntw - 2];
        const int kid = routed ? (gate_up ? MOE_FFN_K_GG_GATE_UP : MOE_FFN_K_GG_DOWN)
                               : (gate_up ? MOE_FFN_K_SH_GATE_UP : MOE_FFN_K_SH_DOWN);
        // a multiple of 8 workgroups keeps job j on XCD j % 8 across the grid-stride loop
        const int grid = std::max(8, expert_grid(jobs, occ) / 8 * 8);
        return timed(P, kid, s, [&] { return launch_pf(g, gate_up, pf_ntw, grid, s); });
    };
    auto run_gg_gate_up = [&](hipStream_t s, bool routed, bool shared) {
        if (pf) return run_pf(s, true, routed, shared);
        GGParams g = gg;
        g.w0 = (const uint8_t *)t->w_gate; g.w1 = (const uint8_t *)t->w_up;
        g.sw0 = (const uint8_t *)t->sh_gate; g.sw1 = (const uint8_t *)t->sh_up;
        g.routed = routed ? 1 : 0;
        g.tiles_routed = (int)((I + gg_rows - 1) / gg_rows);
        g.tiles_shared = shared ? (int)((Is + gg_rows - 1) / gg_rows) : 0;
        const int nt = gg_nt;
        const int jobs = g.tiles_shared * gg_tb + (routed ? max_used * g.tiles_routed : 0);
        const int kid = routed ? MOE_FFN_K_GG_GATE_UP : MOE_FFN_K_SH_GATE_UP;
        return timed(P, kid, s, [&] {
            return launch_gg_gate_up(g, nt, expert_grid(jobs, P->occ_gg_gu[nt_index(nt)]), s);
        });
    };
    auto run_gg_down = [&](hipStream_t s, bool routed, bool shared) {
        if (pf) return run_pf(s, false, routed, shared);
        GGParams g = gg;
        g.w0 = (const uint8_t *)t->w_down; g.sw0 = (const uint8_t *)t->sh_down;
        g.routed = routed ? 1 : 0;
        g.tiles_routed = (int)((H + gg_rows - 1) / gg_rows);
        g.tiles_shared = shared ? g.tiles_routed : 0;
        const int nt = gg_nt;
        const int jobs = g.tiles_shared * gg_tb + (routed ? max_used * g.tiles_routed : 0);
        const int kid = routed ? MOE_FFN_K_GG_DOWN : MOE_FFN_K_SH_DOWN;
        return timed(P, kid, s, [&] {
            return launch_gg_down(g, nt, expert_grid(jobs, P->occ_gg_d[nt_index(nt)]), s);
        });
    };
    // one step of the layer in the regime of this call
    auto step_gate_up = [&](hipStream_t s, bool routed, bool shared) {
        return gemm ? run_gg_gate_up(s, routed, shared) : run_gate_up(s, routed, shared);
    };
    auto step_down = [&](hipStream_t s, bool routed, bool shared) {
        return gemm ? run_gg_down(s, routed, shared) : run_down(s, routed, shared);
    };
    auto run_join = [&](hipStream_t s) {
        return timed(P, MOE_FFN_K_JOIN, s, [&] { return launch_join(jp, s); });
    };

    hipError_t err = hipSuccess;
    auto chk = [&](hipError_t x) {
        if (err == hipSuccess && x != hipSuccess) err = x;
    };
    // the routed down step and the join: one launch (k_down_join) or two
    auto run_tail = [&](hipStream_t s, bool shared_here) {
        if (!use_dj) {
            hipError_t e1 = step_down(s, true, shared_here);
            if (e1 != hipSuccess) return e1;
            return run_join(s);
        }
        DownJoinParams q = djp;
        q.shared_here = shared_here ? 1 : 0;
        return timed(P, MOE_FFN_K_DOWN_JOIN, s, [&] { return launch_down_join(q, wk, P->map_down, s); });
    };
    if (mode == MOE_FFN_SHARED_AUX) {
        // the shared branch reads the experts' input: with the input norm it forks
        // after the router launch that writes it, else at entry
        if (norm) {
            if (delay_main) chk(launch_delay(stream, delay_ticks));
            chk(run_router(stream));
        }
        chk(hipEventRecord(P->ev_fork, stream));
        chk(hipStreamWaitEvent(P->aux, P->ev_fork, 0));
        if (delay_aux) chk(launch_delay(P->aux, delay_ticks));
        chk(step_gate_up(P->aux, false, true));
        chk(step_down(P->aux, false, true));
        chk(hipEventRecord(P->ev_join, P->aux));
        if (!norm) {
            if (delay_main) chk(launch_delay(stream, delay_ticks));
            chk(run_router(stream));
        }
        chk(step_gate_up(stream, true, false));
        if (use_dj) {  // the fused launch reads S: wait for the shared branch first
            chk(hipStreamWaitEvent(stream, P->ev_join, 0));
            chk(run_tail(stream, false));
        } else {
            chk(step_down(stream, true, false));
            chk(hipStreamWaitEvent(stream, P->ev_join, 0));
            chk(run_join(stream));
        }
    } else if (mode == MOE_FFN_SHARED_SEQ) {
        if (norm) chk(run_router(stream));  // writes the experts' input
        if (delay_aux) chk(launch_delay(stream, delay_ticks));
        chk(step_gate_up(stream, false, true));
        chk(step_down(stream, false, true));
        if (delay_main) chk(launch_delay(stream, delay_ticks));
        if (!norm) chk(run_router(stream));
        chk(step_gate_up(stream, true, false));
        chk(run_tail(stream, false));
    } else {  // FUSED
        if (delay_main || delay_aux) chk(launch_delay(stream, delay_ticks));
        chk(run_router(stream));
        chk(step_gate_up(stream, true, true));
        chk(run_tail(stream, true));
    }
    if (err != hipSuccess) return hip_fail(err, "kernel launch");
    if ((err = hipGetLastError()) != hipSuccess) return hip_fail(err, "kernel launch");
    return MOE_FFN_OK;
}

void moe_ffn_destroy(moe_ffn_plan_t P) {
    if (!P) return;
    if (P->aux) hipStreamSynchronize(P->aux);
    for (auto &r : P->prof) {
        hipEventSynchronize(r.stop);
        hipEventDestroy(r.start);
        hipEventDestroy(r.stop);
    }
    for (hipEvent_t e : P->pool) hipEventDestroy(e);
    if (P->ev_fork) hipEventDestroy(P->ev_fork);
    if (P->ev_join) hipEventDestroy(P->ev_join);
    if (P->aux) hipStreamDestroy(P->aux);
    delete P;
}

moe_ffn_status moe_ffn_profile_enable(moe_ffn_plan_t P, int32_t enable) {
    if (!P) return set_error(MOE_FFN_ERR_INVALID_ARG, "plan must not be NULL");
    P->profiling = enable != 0;
    return MOE_FFN_OK;
}

moe_ffn_status moe_ffn_profile_read(moe_ffn_plan_t P, double *total_ms, int64_t *launches) {
    if (!P || !total_ms || !launches) return set_error(MOE_FFN_ERR_INVALID_ARG, "NULL argument");
    for (int i = 0; i < MOE_FFN_K_COUNT; ++i) {
        total_ms[i] = 0.0;
        launches[i] = 0;
    }
    moe_ffn_status st = MOE_FFN_OK;
    for (auto &r : P->prof) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess && st == MOE_FFN_OK) st = hip_fail(e, "hipEventElapsedTime");
        total_ms[r.kernel] += ms;
        launches[r.kernel] += 1;
        P->pool.push_back(r.start);
        P->pool.push_back(r.stop);
    }
    P->prof.clear();
    return st;
}

}  // extern "C"

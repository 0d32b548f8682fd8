// plan.cpp -- host-only planning for the MoE decode FFN layer: validation,
// kernel geometry and the workspace layout.  No HIP runtime call is made here
// (planning may run before any device work exists: page "ggml operator
// extensions", section "Kernel selection", the prepare step).
#include <algorithm>
#include <cstring>
#include <new>
#include <string>

#include "internal.h"

namespace moeffn {

static thread_local std::string g_last_error;

moe_ffn_status set_error(moe_ffn_status st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

size_t row_bytes_of(int wkind, int k_elems) {
    switch (wkind) {
    case W_F32: return (size_t)k_elems * 4;
    case W_BF16: return (size_t)k_elems * 2;
    default: return (size_t)k_elems / 2;  // W_Q4 (scales live in their own tensor)
    }
}

static int pow2_ceil(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

RowMap make_row_map(size_t row_bytes) {
    RowMap m;
    m.n_chunks = (int)(row_bytes / 16);
    if (m.n_chunks >= 64) {
        m.lpr = 64;
        m.nc = pow2_ceil((m.n_chunks + 63) / 64);
    } else {
        m.lpr = std::max(8, pow2_ceil(m.n_chunks));
        m.nc = 1;
    }
    return m;
}

static size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

}  // namespace moeffn

using namespace moeffn;

extern "C" {

int32_t moe_ffn_abi_version(void) { return MOE_FFN_ABI_VERSION; }

const char *moe_ffn_last_error(void) { return g_last_error.c_str(); }

const char *moe_ffn_status_string(int32_t status) {
    switch (status) {
    case MOE_FFN_OK: return "ok";
    case MOE_FFN_ERR_INVALID_ARG: return "invalid argument";
    case MOE_FFN_ERR_UNSUPPORTED: return "unsupported";
    case MOE_FFN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_FFN_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_FFN_ERR_ALIAS: return "output overlaps an input";
    case MOE_FFN_ERR_TOO_MANY_TOKENS: return "token count out of range";
    case MOE_FFN_ERR_HIP: return "HIP runtime error";
    case MOE_FFN_ERR_WRONG_DEVICE: return "wrong device";
    default: return "unknown status";
    }
}

size_t moe_ffn_struct_size(int32_t which) {
    switch (which) {
    case 0: return sizeof(moe_ffn_desc);
    case 1: return sizeof(moe_ffn_tensors);
    case 2: return sizeof(moe_ffn_plan_info);
    case 3: return sizeof(moe_ffn_routing_layout);
    default: return 0;
    }
}

moe_ffn_status moe_ffn_plan(const moe_ffn_desc *desc, moe_ffn_plan_t *out_plan,
                            size_t *workspace_bytes) {
    if (out_plan) *out_plan = nullptr;
    if (!desc || !out_plan) return set_error(MOE_FFN_ERR_INVALID_ARG, "desc and out_plan must not be NULL");
    const moe_ffn_desc d = *desc;
    const uint32_t known = MOE_FFN_SHARED_MASK | MOE_FFN_FORCE_MATVEC | MOE_FFN_FORCE_GEMM |
                           MOE_FFN_DEBUG_DELAY_AUX | MOE_FFN_DEBUG_DELAY_MAIN | MOE_FFN_DEBUG_SPLIT_JOIN |
                           MOE_FFN_INPUT_NORM | MOE_FFN_RESIDUAL;
    if (d.flags & ~known) return set_error(MOE_FFN_ERR_INVALID_ARG, "unknown flag bits");
    if ((d.flags & MOE_FFN_INPUT_NORM) && !(d.norm_eps >= 0.f && d.norm_eps <= 3.4e38f))
        return set_error(MOE_FFN_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
    if ((d.flags & MOE_FFN_FORCE_MATVEC) && (d.flags & MOE_FFN_FORCE_GEMM))
        return set_error(MOE_FFN_ERR_INVALID_ARG, "FORCE_MATVEC and FORCE_GEMM are exclusive");
    if (d.hidden <= 0 || d.n_experts <= 0 || d.top_k <= 0 || d.inter <= 0 || d.shared_inter <= 0 ||
        d.max_tokens <= 0 || d.device < 0 || d.matvec_max_tokens < 0)
        return set_error(MOE_FFN_ERR_INVALID_ARG, "sizes must be positive (device, matvec_max_tokens >= 0)");
    if (d.top_k > d.n_experts) return set_error(MOE_FFN_ERR_INVALID_ARG, "top_k > n_experts");
    if (d.x_dtype < MOE_FFN_F32 || d.x_dtype > MOE_FFN_BF16 || d.weight_dtype < MOE_FFN_F32 ||
        d.weight_dtype > MOE_FFN_Q4_B32)
        return set_error(MOE_FFN_ERR_INVALID_ARG, "unknown dtype");
    for (int v : {d.hidden, d.inter, d.shared_inter})
        if (v % 32 != 0 || v > kMaxDim)
            return set_error(MOE_FFN_ERR_UNSUPPORTED, "hidden/inter/shared_inter must be multiples of 32, at most 8192");
    if (d.n_experts > kMaxExperts) return set_error(MOE_FFN_ERR_UNSUPPORTED, "n_experts > 512");
    if (d.top_k > kMaxTopK) return set_error(MOE_FFN_ERR_UNSUPPORTED, "top_k > 32");
    if (d.max_tokens > kMaxTokens) return set_error(MOE_FFN_ERR_UNSUPPORTED, "max_tokens > 16384");
    const bool pair_ok = (d.x_dtype == MOE_FFN_F32 && d.weight_dtype == MOE_FFN_F32) ||
                         (d.x_dtype == MOE_FFN_BF16 && d.weight_dtype == MOE_FFN_BF16) ||
                         (d.x_dtype == MOE_FFN_BF16 && d.weight_dtype == MOE_FFN_Q4_B32);
    if (!pair_ok) return set_error(MOE_FFN_ERR_UNSUPPORTED, "unsupported (x_dtype, weight_dtype) pair");
    // the grouped MFMA GEMM takes bf16 weights and tokens, K in chunks of 128, rows in 64s
    const bool gemm_ok = d.weight_dtype == MOE_FFN_BF16 && d.x_dtype == MOE_FFN_BF16 &&
                         d.hidden % 128 == 0 && d.inter % 128 == 0 && d.shared_inter % 128 == 0;
    if ((d.flags & MOE_FFN_FORCE_GEMM) && !gemm_ok)
        return set_error(MOE_FFN_ERR_UNSUPPORTED,
                         "the grouped-GEMM regime needs bf16 weights and tokens and sizes that are multiples of 128");

    moe_ffn_plan_s *P = new (std::nothrow) moe_ffn_plan_s;
    if (!P) return set_error(MOE_FFN_ERR_INVALID_ARG, "out of host memory");
    P->d = d;
    P->wkind = d.weight_dtype;
    P->gemm_ok = gemm_ok && !(d.flags & MOE_FFN_FORCE_MATVEC);
    // regime threshold: mat-vec kernels up to it, grouped MFMA GEMM above (bf16
    // storage).  AUTO folds the shared expert into the routed launches in both
    // regimes: measured faster than the second stream at every batch tried
    P->matvec_max = d.matvec_max_tokens ? d.matvec_max_tokens : kDefaultMatvecMax;
    const uint32_t mode = d.flags & MOE_FFN_SHARED_MASK;
    P->mode_matvec = mode == MOE_FFN_SHARED_AUTO ? MOE_FFN_SHARED_FUSED : mode;
    P->mode_gemm = mode == MOE_FFN_SHARED_AUTO ? MOE_FFN_SHARED_FUSED : mode;

    const int H = d.hidden, E = d.n_experts, k = d.top_k, I = d.inter, Is = d.shared_inter;
    const size_t T = (size_t)d.max_tokens, P_ = T * k;
    P->map_gu = make_row_map(row_bytes_of(P->wkind, H));
    P->map_down = make_row_map(row_bytes_of(P->wkind, std::max(I, Is)));

    // LDS of each kernel at the largest batch it can see
    const int xbytes = d.x_dtype == MOE_FFN_F32 ? 4 : 2;
    RouterParams rq{};
    rq.H = H; rq.x_bf16 = xbytes == 2;
    rq.tok_tile = std::max(1, std::min(8, (int)(kStageBytes / ((size_t)H * xbytes))));
    const bool maps_ok = P->map_gu.nc <= 16 && P->map_down.nc <= 16 && router_chunks_per_lane(H) <= 8;
    if (!maps_ok || router_lds_bytes(rq) > kLdsLimit) {
        delete P;
        return set_error(MOE_FFN_ERR_UNSUPPORTED, "shapes exceed the per-workgroup LDS budget");
    }

    // the routing launch ranks and buckets up to kRouteKernelMax tokens in LDS; where
    // that does not fit (many experts and picks), those batches take batch routing too
    const bool route_fits = route_kernel_lds_bytes(std::min(d.max_tokens, kRouteKernelMax), k, E) <= kLdsLimit;

    Layout &L = P->L;
    size_t c = 0;
    L.sh_h = c;       c += align_up(T * Is * 4);
    L.sh_S = c;       c += align_up(T * H * 4);
    L.shared_bytes = c;
    L.gate_s = c;     c += align_up(T * 4);
    L.ids = c;        c += align_up(P_ * 4);
    L.wts = c;        c += align_up(P_ * 4);
    L.records = c;    c += align_up((size_t)E * kRecInts * 4);
    L.n_unique = c;   c += align_up(16);
    L.pairs = c;      c += align_up(P_ * 4);
    L.pos_expert = c; c += align_up(P_ * 4);
    L.logits = c;     c += align_up(T * logit_stride(E) * 4);
    // normalised input of both branches (x_dtype), router -> experts
    L.xn = c;         c += (d.flags & MOE_FFN_INPUT_NORM) ? align_up(T * H * xbytes) : 0;
    // batch routing's counts, prefixes and ranks (batches above kRouteKernelMax)
    const bool batch_possible = d.max_tokens > kRouteKernelMax || !route_fits;
    L.bcount = c;     c += batch_possible ? align_up(batch_route_ints(d.max_tokens, k, E) * 4) : 0;
    L.routing_bytes = c - L.shared_bytes;
    // sequential steps: gate/up holds h, down holds h and y, join holds y
    const size_t base = c;
    const size_t hb = align_up(P_ * I * 4), yb = align_up(P_ * H * 4);
    L.h = base;
    L.y = base + hb;
    L.phase_bytes = std::max({hb, hb + yb, yb});
    L.total = base + L.phase_bytes;

    *out_plan = P;
    if (workspace_bytes) *workspace_bytes = L.total;
    return MOE_FFN_OK;
}

moe_ffn_status moe_ffn_plan_get_info(moe_ffn_plan_t plan, moe_ffn_plan_info *info) {
    if (!plan || !info) return set_error(MOE_FFN_ERR_INVALID_ARG, "plan and info must not be NULL");
    info->workspace_bytes = plan->L.total;
    info->shared_region_bytes = plan->L.shared_bytes;
    info->routing_region_bytes = plan->L.routing_bytes;
    info->phase_region_bytes = plan->L.phase_bytes;
    info->matvec_max_tokens = plan->matvec_max;
    info->shared_mode_matvec = plan->mode_matvec;
    info->shared_mode_gemm = plan->mode_gemm;
    return MOE_FFN_OK;
}

moe_ffn_status moe_ffn_plan_get_routing_layout(moe_ffn_plan_t plan, moe_ffn_routing_layout *layout) {
    if (!plan || !layout) return set_error(MOE_FFN_ERR_INVALID_ARG, "plan and layout must not be NULL");
    const Layout &L = plan->L;
    layout->ids = L.ids;
    layout->weights = L.wts;
    layout->gate = L.gate_s;
    layout->n_used = L.n_unique;
    layout->records = L.records;
    layout->pairs = L.pairs;
    layout->pair_expert = L.pos_expert;
    layout->record_ints = kRecInts;
    layout->record_pairs = kRecPairs;
    return MOE_FFN_OK;
}

}  // extern "C"

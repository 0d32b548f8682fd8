// internal.h -- host-side structures shared by the planner, the launcher and
// the kernel files of the MoE decode FFN library (not part of the ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "moe_ffn.h"

namespace moeffn {

constexpr int kMaxTokens = 16384;
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 32;
constexpr int kMaxDim = 8192;
constexpr int kDefaultMatvecMax = 16;  // measured crossover of the mat-vec and grouped-GEMM kernels
constexpr int kRouteInGateUpMax = 16;  // up to this batch the gate/up workgroups route it themselves
constexpr int kRouteKernelMax = 16;   // up to this batch k_route routes it (else the batch launches)
constexpr int kPfMinBucket = 32;      // mean tokens per used expert from which the prefill GEMM runs
constexpr size_t kWsAlign = 256;
constexpr size_t kLdsLimit = 64 * 1024;   // dynamic LDS per workgroup used by any kernel
constexpr size_t kStageBytes = 32 * 1024; // activation staging per workgroup

// Floats per token row of the logits table: E router logits, the shared-gate logit
// at column E, padded to a multiple of 4 so that each row starts 16-byte aligned and
// a lane reads four logits with one load.
__host__ __device__ constexpr int logit_stride(int E) { return (E + 1 + 3) / 4 * 4; }

// weight storage as the kernels see it
enum WKind : int { W_F32 = 0, W_BF16 = 1, W_Q4 = 2 };

// How a 16-byte-chunked row maps onto a wave: LPR lanes per row, NC chunks
// per lane (chunk c of a row is read by lane c % LPR of the row's segment).
struct RowMap {
    int lpr = 64;
    int nc = 1;
    int n_chunks = 0;  // 16-byte chunks in one row
};

// Workspace layout: byte offsets from the workspace base, kWsAlign-aligned.
struct Layout {
    // shared-branch region (written only by the shared branch)
    size_t sh_h = 0;    // f32 [Tmax][Is]
    size_t sh_S = 0;    // f32 [Tmax][H]
    size_t shared_bytes = 0;
    // routing region (router -> join)
    size_t gate_s = 0;     // f32 [Tmax]
    size_t ids = 0;        // i32 [Tmax*k]
    size_t wts = 0;        // f32 [Tmax*k]
    size_t records = 0;    // i32 [E][kRecInts]: job record per used expert
    size_t n_unique = 0;   // i32 [4]
    size_t pairs = 0;      // i32 [Tmax*k]: pair id t*k+j in expert-bucketed order
    size_t pos_expert = 0; // i32 [Tmax*k]: expert of each bucketed position
    size_t logits = 0;     // f32 [Tmax][E+1] (column E = shared-gate logit), router -> gate/up
    size_t xn = 0;         // x_dtype [Tmax][H]: normalised input (INPUT_NORM), router -> experts
    size_t bcount = 0;     // i32: batch routing's totals [E], count rows [W][E], in-workgroup ranks [T*k]
    size_t routing_bytes = 0;
    // phase region: reused by the sequential steps
    size_t h = 0;       // gate/up -> down: f32 [Tmax*k][I]
    size_t y = 0;       // down -> join: f32 [Tmax*k][H] (live together with h during down)
    size_t phase_bytes = 0;
    size_t total = 0;
};

struct ProfRec {
    int kernel;
    hipEvent_t start, stop;
};

}  // namespace moeffn

struct moe_ffn_plan_s {
    moe_ffn_desc d{};
    moeffn::Layout L{};
    int matvec_max = 0;
    uint32_t mode_matvec = MOE_FFN_SHARED_FUSED;
    uint32_t mode_gemm = MOE_FFN_SHARED_SEQ;
    int wkind = 0;
    // row maps: router rows (fp32, K=H), gate/up rows (K=H), down rows (K=max(I,Is))
    moeffn::RowMap map_gu, map_down;
    // lazily created device state
    bool ready = false;
    hipStream_t aux = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    int cu_count = 0;       // compute units of the device
    int occ_gu = 0, occ_d = 0;  // resident workgroups per CU of the expert kernels
    int occ_gu1 = 0;            // the same for the one-row-per-wave gate/up kernel
    int occ_gg_gu[3] = {0, 0, 0}, occ_gg_d[3] = {0, 0, 0};  // grouped GEMM, 16/32/64 tokens per pass
    int occ_pf_gu[3] = {0, 0, 0}, occ_pf_d[3] = {0, 0, 0};  // prefill GEMM, 128/192/256 tokens per pass
    bool gemm_ok = false;   // shapes and storage the grouped GEMM supports
    // profiling
    bool profiling = false;
    std::vector<moeffn::ProfRec> prof;
    std::vector<hipEvent_t> pool;
};

namespace moeffn {

// ---- kernel launch parameter blocks ---------------------------------------

// A job record per used expert: expert, first bucketed position, token count,
// 0, then the first kRecPairs pair ids (t*k + j) of its bucket (-1 past count).
constexpr int kRecInts = 16;
constexpr int kRecPairs = kRecInts - 4;

struct RouterParams {
    const void *x;
    int x_bf16;
    int T, H, E, k;
    const float *router;    // [E][H]
    const float *gate_vec;  // [H] (acts as row E)
    float *logits;          // [T][E+1]
    int tok_tile;           // tokens per workgroup column
    // routing outputs (written by the last workgroup of each token tile / of the launch)
    int *ids;               // [T*k]
    float *wts;             // [T*k]
    float *gate_s;          // [T]
    int *records;           // [E][kRecInts]
    int *n_unique;          // [1]
    int *pairs;             // [T*k]
    int *pos_expert;        // [T*k]
    int32_t *dbg_ids;
    float *dbg_w, *dbg_logits, *dbg_gate;
    // input RMSNorm: logits from the normalised tokens; workgroup column 0 writes them for the experts
    const float *norm_w;    // [H] or NULL: no norm
    float norm_eps;
    void *xn;               // [T][H] x_dtype
    // batch routing (large batches): k_rank_batch ranks and counts per workgroup,
    // k_count_scan turns the counts into prefixes, k_bucket_batch places the pairs
    int *bcount;            // totals [E], count rows [W][E], in-workgroup ranks [T*k]; or NULL
};

struct GateUpParams {
    const void *x;
    int T, H, k, E;
    int x_resident;                // 1: all T tokens staged in LDS once
    int tok_per_pass;              // else: tokens staged per pass
    int x_sums;                    // 1 (4-bit weights): the stage also holds each 32-element
                                   // block's sum of activations, after the tokens
    // routed experts
    const uint8_t *wg, *wu;        // [E][I] rows
    const uint16_t *sg, *su;       // Q4 scales [E][I][H/32]
    int I;
    const int *records;
    const int *n_unique;
    const int *pairs;
    float *h;                      // [T*k][I]
    int routed;                    // routed experts' jobs are in this launch
    int tiles_routed;              // jobs per routed expert
    // shared expert
    const uint8_t *swg, *swu;
    const uint16_t *ssg, *ssu;
    int Is;
    float *hs;                     // [T][Is]
    int tiles_shared;              // jobs of the shared expert (0 = not in this launch)
    // routing in every workgroup (small batches; routed launches only)
    int route_here;                // 1: rank and bucket the batch from the logits here
    int route_lds_off;             // byte offset of the routing area in dynamic LDS
    const float *logits;           // [T][E+1]
    int *ids;                      // global tables, written by workgroup 0
    float *wts;
    float *gate_s;
    int *pos_expert;
    int32_t *dbg_ids;
    float *dbg_w, *dbg_logits, *dbg_gate;
};

struct DownParams {
    int T, H, k, E;
    // routed experts
    const uint8_t *wd;   // [E][H] rows of I
    const uint16_t *sd;  // [E][H][I/32]
    int I;
    const float *h;      // [T*k][I]
    const int *records;
    const int *n_unique;
    const int *pairs;
    float *y;            // [T*k][H]
    int routed;
    int tiles_routed;
    // shared expert
    const uint8_t *swd;  // [H] rows of Is
    const uint16_t *ssd; // [H][Is/32]
    int Is;
    const float *hs;     // [T][Is]
    float *S;            // [T][H]
    int tiles_shared;
};

struct DownJoinParams {
    int T, H, k, E;
    const uint8_t *wd;      // [E][H] rows of I
    const uint16_t *sd;     // [E][H][I/32]
    int I;
    const float *h;         // [T*k][I]
    const int *pairs;       // [T*k] bucketed order
    const int *pos_expert;  // [T*k]
    const uint8_t *swd;     // [H] rows of Is
    const uint16_t *ssd;
    int Is;
    const float *hs;        // [T][Is]
    int shared_here;        // 1: the shared expert's down runs here; 0: S comes from memory
    const float *S;         // [T][H] (shared_here == 0)
    const float *wts;       // [T*k]
    const float *gate_s;    // [T]
    float *out;             // [T][H]
    const void *resid;      // [T][H] x_dtype: the residual input, or NULL
    int resid_bf16;
};

struct GGParams {
    const void *x;       // [T][H] bf16
    int T, H, k, E, I, Is;
    const uint8_t *w0, *w1;    // routed: gate and up [E][I][H] (gate/up launch) or down [E][H][I]
    const uint8_t *sw0, *sw1;  // shared: gate and up [Is][H] or down [H][Is]
    const int *records;
    const int *n_unique;
    const int *pairs;
    uint16_t *hb;        // [T*k][I] bf16
    uint16_t *shb;       // [T][Is] bf16
    float *y;            // [T*k][H]
    float *S;            // [T][H]
    int routed, tiles_routed, tiles_shared;
};

struct JoinParams {
    const void *resid;   // [T][H] x_dtype: the residual input, or NULL
    int resid_bf16;
    int T, H, k;
    const float *y;      // [T*k][H]
    const float *wts;    // [T*k]
    const float *gate_s; // [T]
    const float *S;      // [T][H]
    float *out;          // [T][H]
};

// ---- profiling: events the next kernel launch records around itself ------
// Set by the forward's timing wrapper; the launch puts them into its own
// dispatch (start and end timestamps of the kernel itself) and clears them.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;

template <typename K, typename... A>
inline void launch_kernel(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, A... args) {
    if (g_launch_events.start) {
        const LaunchEvents ev = g_launch_events;
        g_launch_events = LaunchEvents{};
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    }
}

// ---- launchers (kernel files) -------------------------------------------
hipError_t launch_router(const RouterParams &p, int grid_tiles, hipStream_t s);
int router_chunks_per_lane(int H);
hipError_t launch_gate_up(const GateUpParams &p, int wkind, const RowMap &m, int grid, hipStream_t s);
hipError_t launch_down(const DownParams &p, int wkind, const RowMap &m, int grid, hipStream_t s);
hipError_t launch_join(const JoinParams &p, hipStream_t s);
hipError_t launch_down_join(const DownJoinParams &p, int wkind, const RowMap &m, hipStream_t s);
int down_join_rows_per_wg(const RowMap &m);
size_t down_join_lds_bytes(int T, int k, const RowMap &m);
hipError_t launch_gg_gate_up(const GGParams &p, int nt, int grid, hipStream_t s);
hipError_t launch_gg_down(const GGParams &p, int nt, int grid, hipStream_t s);
int gg_occupancy(bool gate_up, int nt);
int gg_rows_per_job();
hipError_t launch_delay(hipStream_t s, uint64_t ticks);

// rows each workgroup covers for a kernel family and row map
int gate_up_rows_per_wg(int wkind, const RowMap &m, int T, bool route_here);
bool gate_up_one_row(int wkind, const RowMap &m, int T, bool route_here);
int gate_up_one_row_occupancy(const RowMap &m, size_t lds);
int down_rows_per_wg(int wkind, const RowMap &m);
size_t gate_up_lds_bytes(const GateUpParams &p, int xbytes);
int gate_up_route_lds_off(const GateUpParams &p, int xbytes);
size_t router_lds_bytes(const RouterParams &p);
size_t route_kernel_lds_bytes(int T, int k, int E);
hipError_t launch_route(const RouterParams &p, hipStream_t s);
hipError_t launch_rank_batch(const RouterParams &p, hipStream_t s);
hipError_t launch_count_scan(const RouterParams &p, hipStream_t s);
size_t batch_route_ints(int T, int k, int E);
hipError_t launch_router_mfma(const RouterParams &p, hipStream_t s);
// prefill grouped GEMM (large buckets)
size_t pf_lds_bytes();
int pf_rows_per_job(bool gate_up);
int pf_tokens_per_pass(int ntw);
hipError_t launch_pf(const GGParams &p, bool gate_up, int ntw, int grid, hipStream_t s);
int pf_occupancy(bool gate_up, int ntw);
int pf_job_count(int tiles_shared, int n_tb, int nu, int tiles_routed);
hipError_t launch_bucket_batch(const RouterParams &p, hipStream_t s);
int expert_kernel_occupancy(bool gate_up, int wkind, const RowMap &m, size_t lds);

// ---- planner helpers (plan.cpp) ---------------------------------------------
RowMap make_row_map(size_t row_bytes);
size_t row_bytes_of(int wkind, int k_elems);
moe_ffn_status set_error(moe_ffn_status st, const std::string &msg);

}  // namespace moeffn

/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) decode-step MoE feed-forward
 * layer with a gated shared expert.
 *
 * The layer (per token x, all arithmetic fp32 on the GPU):
 *   logits  l = Wr x                          (router, E rows)
 *   ids     the k largest logits, ties to the lower expert index, rank order
 *   weights w_j = softmax(l)[ids_j] / sum_j' softmax(l)[ids_j']
 *   routed  r = sum_j w_j Wd[ids_j] (silu(Wg[ids_j] x) * (Wu[ids_j] x))
 *   shared  S = Ws_d (silu(Ws_g x) * (Ws_u x)),  s = sigmoid(w_gate . x)
 *   out     = r + s*S   (the product and the sum rounded separately)
 * Structure: routed experts plus one gated shared expert, joined by a final
 * add -- page "ggml-cuda: overlap the MoE shared expert on a separate stream",
 * section "What this changes".  SwiGLU with separate gate and up matrices --
 * page "ggml operator extensions", section "sd.cpp integration".
 *
 * Lifecycle (page "ggml operator extensions", section "Kernel selection": a
 * prepare step that only plans and sizes workspace, an execute step that gets
 * the stream, workspace and current addresses, and a destroy step):
 *   moe_ffn_plan     host only: validates shapes, picks kernels, sizes ONE
 *                    workspace; no HIP call, no device allocation, no launch.
 *   moe_ffn_forward  enqueues the layer on the caller's stream and returns.
 *   moe_ffn_destroy  releases the plan (NULL is a no-op).
 *
 * Ownership: the caller owns every tensor, the workspace and the stream; the
 * library borrows them for the duration of the enqueued work (same page,
 * section "Backend services": borrowed device and stream, ordered with the
 * caller's work).  The plan owns no device memory.  A plan whose shared-expert
 * mode uses the second stream (MOE_FFN_SHARED_AUX) owns that HIP stream and two
 * events, created lazily by its first forward; every plan queries the device
 * (compute units, kernel occupancy) in its first forward, which therefore must
 * not run under stream capture.
 *
 * Threading: a plan serialises nothing.  Two forwards of one plan must not
 * run concurrently (they share the plan's stream and usually the workspace).
 * Plans are independent of each other.
 *
 * Errors: every entry point validates before it enqueues anything and returns
 * a specific status; it never retries and never switches to another algorithm
 * on failure (same page, section "Kernel selection": errors propagate and a
 * native path is never retried after launch).  moe_ffn_last_error() gives a
 * human-readable reason for the last failure on the calling thread.  No C++
 * exception crosses this ABI.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_ABI_VERSION 2

typedef enum moe_ffn_status {
    MOE_FFN_OK = 0,
    MOE_FFN_ERR_INVALID_ARG = 1,          /* NULL where required, inconsistent shapes, unknown enum */
    MOE_FFN_ERR_UNSUPPORTED = 2,          /* valid but outside the limits below, or first forward under capture */
    MOE_FFN_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below what the plan reported */
    MOE_FFN_ERR_MISALIGNED = 4,           /* a tensor not 16-byte aligned, or the workspace not 256-byte aligned */
    MOE_FFN_ERR_ALIAS = 5,                /* out overlaps an input other than by exact equality with x */
    MOE_FFN_ERR_TOO_MANY_TOKENS = 6,      /* n_tokens < 0 or > desc.max_tokens */
    MOE_FFN_ERR_HIP = 7,                  /* a HIP runtime call or kernel launch failed */
    MOE_FFN_ERR_WRONG_DEVICE = 8          /* current device or stream's device differs from desc.device */
} moe_ffn_status;

typedef enum moe_ffn_dtype {
    MOE_FFN_F32 = 0,
    MOE_FFN_BF16 = 1,
    /* 4-bit symmetric blocks: 32 consecutive elements along a row's reduction
     * dimension form a block; element c of the row is in byte c/2, low nibble
     * for even c, high nibble for odd c, stored as u = q + 8 (q in [-8, 7]);
     * its value is scale[row][c/32] * q with one fp16 scale per block in a
     * separate tensor. */
    MOE_FFN_Q4_B32 = 2
} moe_ffn_dtype;

/* desc.flags ---------------------------------------------------------------
 * Where the shared expert runs (page "ggml-cuda: overlap the MoE shared
 * expert on a separate stream", section "What this changes": the shared
 * expert forked onto one auxiliary stream and joined at the add, only in the
 * small-batch mat-vec regime, output identical to sequential order).  Every
 * mode gives bit-identical output for the same inputs. */
#define MOE_FFN_SHARED_AUTO 0x0u   /* FUSED in both regimes (measured fastest; moe_ffn_plan_info) */
#define MOE_FFN_SHARED_AUX 0x1u    /* second stream of the plan, event fork at entry, event join before the add */
#define MOE_FFN_SHARED_SEQ 0x2u    /* same kernels, all on the caller's stream, shared branch first */
#define MOE_FFN_SHARED_FUSED 0x3u  /* shared expert folded into the routed kernels' grids (fewest launches) */
#define MOE_FFN_SHARED_MASK 0x3u
/* Regime: mat-vec kernels while n_tokens <= desc.matvec_max_tokens, grouped
 * MFMA GEMM above it where the storage is (BF16, BF16) with hidden, inter and
 * shared_inter multiples of 128 (other storage stays on the mat-vec kernels).
 * The FORCE flags pin one regime for every n_tokens; FORCE_GEMM on storage the
 * GEMM does not take is MOE_FFN_ERR_UNSUPPORTED at planning.  The GEMM regime
 * rounds the SwiGLU activation to bf16 before the down product; the mat-vec
 * regime keeps it in fp32.  The shared-expert modes agree bit for bit within
 * a regime. */
#define MOE_FFN_FORCE_MATVEC 0x10u
#define MOE_FFN_FORCE_GEMM 0x20u
/* Test hooks: a bounded (about 200 us) spin kernel at the head of the aux
 * branch or of the main branch, to expose a missing wait or a launch on the
 * wrong stream.  They change timing only, never results. */
#define MOE_FFN_DEBUG_DELAY_AUX 0x100u
#define MOE_FFN_DEBUG_DELAY_MAIN 0x200u
/* The decode block around the layer (page "ggml-cuda: overlap the MoE shared
 * expert on a separate stream", its commit list: the FFN-input norm is the node
 * both branches fork from, and the branches meet at an add; page "ggml operator
 * extensions", section "sd.cpp integration": an RMSNorm followed by a multiply
 * with a one-dimensional weight vector; each operation rounded separately):
 *   INPUT_NORM  x -> (x * rho) * norm_weight, rho = 1/sqrt(mean(x^2) + norm_eps),
 *               per token in fp32; the router takes it in fp32, the experts and
 *               the shared expert in x_dtype (bf16 x: rounded to nearest even).
 *   RESIDUAL    out = x + (routed + s * S), x the layer's input before any norm,
 *               each operation rounded to fp32 separately. */
#define MOE_FFN_INPUT_NORM 0x1000u
#define MOE_FFN_RESIDUAL 0x2000u
/* Test hook: in the mat-vec regime run the down step and the join as two
 * launches where one (MOE_FFN_K_DOWN_JOIN) would apply.  Results are
 * bit-identical either way. */
#define MOE_FFN_DEBUG_SPLIT_JOIN 0x400u

/* Shapes and storage; frozen for the life of the plan.
 * Limits (else MOE_FFN_ERR_UNSUPPORTED): hidden, inter, shared_inter
 * multiples of 32 and at most 8192; n_experts 1..512; top_k 1..32 and
 * <= n_experts; max_tokens 1..16384; supported storage pairs (x_dtype,
 * weight_dtype): (F32, F32), (BF16, BF16), (BF16, Q4_B32). */
typedef struct moe_ffn_desc {
    int32_t hidden;             /* H */
    int32_t n_experts;          /* E */
    int32_t top_k;              /* k */
    int32_t inter;              /* I, routed-expert intermediate size */
    int32_t shared_inter;       /* I_s, shared-expert intermediate size */
    int32_t max_tokens;         /* largest n_tokens any forward of this plan may pass */
    int32_t device;             /* HIP device ordinal the plan runs on */
    int32_t x_dtype;            /* moe_ffn_dtype of x: F32 or BF16 */
    int32_t weight_dtype;       /* moe_ffn_dtype of every routed and shared FFN matrix */
    uint32_t flags;             /* MOE_FFN_SHARED_*, MOE_FFN_FORCE_*, MOE_FFN_INPUT_NORM,
                                   MOE_FFN_RESIDUAL, MOE_FFN_DEBUG_* */
    int32_t matvec_max_tokens;  /* regime switch; 0 = library default (16) */
    float norm_eps;             /* INPUT_NORM epsilon (>= 0, finite); ignored otherwise */
} moe_ffn_desc;

/* Device pointers for one forward.  Row-major, contiguous, 16-byte aligned.
 * Weights are in [out, in] orientation.  The router and the gate vector are
 * always fp32.  For Q4_B32 storage a matrix of logical shape [.., R, K] is
 * uint8 [.., R, K/2] plus an fp16 scale tensor [.., R, K/32]; the *_scale
 * pointers must be NULL for other storage. */
typedef struct moe_ffn_tensors {
    const void *x;               /* [T, H] x_dtype */
    const float *w_router;       /* [E, H] */
    const void *w_gate;          /* [E, I, H] */
    const void *w_up;            /* [E, I, H] */
    const void *w_down;          /* [E, H, I] */
    const uint16_t *w_gate_scale;  /* Q4_B32: fp16 [E, I, H/32] */
    const uint16_t *w_up_scale;    /* Q4_B32: fp16 [E, I, H/32] */
    const uint16_t *w_down_scale;  /* Q4_B32: fp16 [E, H, I/32] */
    const void *sh_gate;         /* [I_s, H] */
    const void *sh_up;           /* [I_s, H] */
    const void *sh_down;         /* [H, I_s] */
    const uint16_t *sh_gate_scale; /* Q4_B32: fp16 [I_s, H/32] */
    const uint16_t *sh_up_scale;   /* Q4_B32: fp16 [I_s, H/32] */
    const uint16_t *sh_down_scale; /* Q4_B32: fp16 [H, I_s/32] */
    const float *gate_vec;       /* [H]: s = sigmoid(gate_vec . x) */
    float *out;                  /* [T, H] fp32.  May equal x exactly (F32 x: in place);
                                    any other overlap with an input -> MOE_FFN_ERR_ALIAS */
    /* Optional outputs for tests (NULL = not written). */
    int32_t *dbg_topk_ids;       /* [T, k] expert ids in rank order */
    float *dbg_topk_weights;     /* [T, k] renormalised routing weights */
    float *dbg_logits;           /* [T, E] router logits */
    float *dbg_shared_gate;      /* [T] sigmoid gate of the shared expert */
    const float *norm_weight;    /* [H] fp32: set exactly when desc.flags has INPUT_NORM */
} moe_ffn_tensors;

typedef struct moe_ffn_plan_s *moe_ffn_plan_t;

/* What a plan decided (for tests, logs and the benchmark). */
typedef struct moe_ffn_plan_info {
    size_t workspace_bytes;      /* = shared_region + routing_region + phase_region */
    size_t shared_region_bytes;  /* written only by the shared branch: disjoint from the rest */
    size_t routing_region_bytes; /* routing results, live from the router to the join */
    size_t phase_region_bytes;   /* max over the sequential steps of their scratch, not the sum */
    int32_t matvec_max_tokens;   /* small-batch threshold actually used */
    uint32_t shared_mode_matvec; /* MOE_FFN_SHARED_{AUX,SEQ,FUSED} used for n_tokens <= threshold */
    uint32_t shared_mode_gemm;   /* ... and above it */
} moe_ffn_plan_info;

/* Where a forward leaves the routing step's integer tables in the workspace:
 * byte offsets from the workspace base, each 256-byte aligned.  The bucketing
 * step groups the batch's (token, slot) pairs by expert so that each selected
 * expert's weights are streamed once per call, whatever the number of tokens
 * that chose it (the routed experts of page "ggml-cuda: overlap the MoE shared
 * expert on a separate stream", section "What this changes", run as mat-vecs
 * at small batches).  Pair q = t*k + j is slot j (rank order) of token t.
 * The tables hold the last forward's results once its work on the stream has
 * completed, until the next call that uses the workspace (page "ggml operator
 * extensions", section "Kernel selection": workspace contents are not
 * preserved between calls).  For tests and tools; no forward reads them from
 * a previous call. */
typedef struct moe_ffn_routing_layout {
    size_t ids;           /* int32 [T*k]: expert of pair q, slots in rank order */
    size_t weights;       /* fp32 [T*k]: renormalised routing weight of pair q */
    size_t gate;          /* fp32 [T]: sigmoid gate of the shared expert per token */
    size_t n_used;        /* int32: distinct experts the batch selected (U) */
    size_t records;       /* int32 [U][record_ints]: one job record per used expert:
                             (expert, first bucketed position, pair count, 0, then the
                             first record_pairs pair ids of its bucket, -1 past the count);
                             up to 16 tokens in order of first appearance (record u is the
                             expert of the u-th pair, in pair order, that is the first to
                             pick its expert; for one token, its rank order), above 16
                             tokens experts ascending */
    size_t pairs;         /* int32 [T*k]: pair ids in bucketed order; each expert's bucket
                             is contiguous and holds its pairs in ascending order; buckets
                             laid out with experts ascending (one token: rank order) */
    size_t pair_expert;   /* int32 [T*k]: expert of each bucketed position */
    int32_t record_ints;  /* ints per job record */
    int32_t record_pairs; /* pair ids held in a record */
} moe_ffn_routing_layout;

/* Kernel ids for the profiling hooks. */
typedef enum moe_ffn_kernel_id {
    MOE_FFN_K_ROUTER = 0,       /* router (logits and the shared-gate logit): a GEMV up to 16 tokens
                                   (and for fp32 tokens or with the input norm), an MFMA GEMM
                                   above */
    MOE_FFN_K_ROUTE = 1,        /* routing launch of its own (top-k, renormalisation, bucketing) for
                                   up to 16 tokens whose routing does not fit the routed gate/up
                                   launch (which routes batches of up to 16 tokens itself when the
                                   batch's logits rows and the routing tables fit its LDS); above
                                   16 tokens the ranking launch (top-k, renormalisation,
                                   per-expert counts) */
    MOE_FFN_K_GATE_UP = 2,      /* gate/up + SiLU*up (routed, or routed + shared when fused) */
    MOE_FFN_K_DOWN = 3,         /* down per (token, slot) pair (routed, or + shared when fused) */
    MOE_FFN_K_SH_GATE_UP = 4,   /* gate/up of the shared expert alone (either regime) */
    MOE_FFN_K_SH_DOWN = 5,      /* down of the shared expert alone (either regime) */
    MOE_FFN_K_JOIN = 6,         /* weighted sum over slots + sigmoid-gated shared output (GEMM regime) */
    MOE_FFN_K_GG_GATE_UP = 7,   /* grouped MFMA gate/up (routed, or routed + shared when fused) */
    MOE_FFN_K_GG_DOWN = 8,      /* grouped MFMA down (routed, or routed + shared when fused) */
    MOE_FFN_K_DOWN_JOIN = 9,    /* mat-vec regime: down of every pair of a row tile + the join */
    MOE_FFN_K_BUCKET = 10,      /* above 16 tokens: bucketing of the ranked pairs by expert (two
                                   launches: the per-expert scan of the counts, the placement) */
    MOE_FFN_K_COUNT = 11
} moe_ffn_kernel_id;

int32_t moe_ffn_abi_version(void);

/* Static string for a status code ("unknown status" for other values). */
const char *moe_ffn_status_string(int32_t status);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char *moe_ffn_last_error(void);

/* sizeof(moe_ffn_desc) for which = 0, sizeof(moe_ffn_tensors) for 1,
 * sizeof(moe_ffn_plan_info) for 2, sizeof(moe_ffn_routing_layout) for 3, else 0
 * (lets bindings check their mirrors). */
size_t moe_ffn_struct_size(int32_t which);

/* Validates desc and creates a plan.  Host only: no HIP call.  On success
 * *out_plan is the new plan and *workspace_bytes (if not NULL) the size of the
 * one workspace every forward needs: the shared-branch region (disjoint,
 * because it runs concurrently with the routed steps) plus the routing region
 * plus the maximum, not the sum, of the sequential steps' scratch (page "ggml
 * operator extensions", section "Kernel selection": workspace capacity is the
 * maximum request, contents not preserved between calls).  On failure
 * *out_plan is NULL. */
moe_ffn_status moe_ffn_plan(const moe_ffn_desc *desc, moe_ffn_plan_t *out_plan,
                            size_t *workspace_bytes);

/* Copies the plan's decisions into *info. */
moe_ffn_status moe_ffn_plan_get_info(moe_ffn_plan_t plan, moe_ffn_plan_info *info);

/* Copies the workspace offsets of the routing tables into *layout (host only;
 * MOE_FFN_ERR_INVALID_ARG for a NULL argument). */
moe_ffn_status moe_ffn_plan_get_routing_layout(moe_ffn_plan_t plan, moe_ffn_routing_layout *layout);

/* Enqueues the layer for tokens 0 .. n_tokens-1 on `stream` (a hipStream_t of
 * desc.device; NULL is that device's null stream) and returns without
 * waiting.  The workspace is device memory of at least the planned size,
 * 256-byte aligned, owned by the caller; its contents are not preserved and
 * every byte read is written earlier in the same call.  Private stream work
 * rejoins `stream` before the call's last kernel, so later work on `stream`
 * may reuse the workspace (same page and section: private-stream use must
 * finish before later backend work can touch the workspace).  No host
 * decision depends on tensor contents, so a forward can be captured into a
 * HIP graph and replayed with new contents at the same addresses (page
 * "ggml operator extensions", section "sd.cpp integration": capture-safe
 * kernels, lazy setup in the first ordinary execution).  n_tokens == 0 is
 * MOE_FFN_OK and enqueues nothing. */
moe_ffn_status moe_ffn_forward(moe_ffn_plan_t plan, const moe_ffn_tensors *tensors,
                               int32_t n_tokens, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid allocation): the same
 * forward, with the workspace taken from a static array the library holds on
 * each device (MOE_FFN_NOALLOC_WORKSPACE_BYTES per GPU, held until the process
 * ends) instead of caller memory.  The caller passes inputs and outputs only.
 * A plan whose workspace_bytes exceed the array is rejected with
 * MOE_FFN_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (the decode layer
 * of hidden 2048, 256 experts, top-8, inter 512 fits up to 128 tokens).  It
 * allocates nothing: the first call on a device looks up that device's copy of
 * the array (hipGetSymbolAddress); the plan's own first-forward set-up is that
 * of moe_ffn_forward.  Every call on one GPU, from any plan, shares that GPU's
 * array, which keeps the last call's contents (no call reads them): calls that
 * overlap on one GPU (other streams, other threads) race and give undefined
 * results; serialise them.  Results are bit-identical to moe_ffn_forward's.
 * Other statuses as moe_ffn_forward. */
#define MOE_FFN_NOALLOC_WORKSPACE_BYTES ((size_t)16 << 20)
moe_ffn_status moe_ffn_forward_noalloc(moe_ffn_plan_t plan, const moe_ffn_tensors *tensors,
                                       int32_t n_tokens, hipStream_t stream);

/* Releases the plan, its stream and events (waits for the plan's own stream
 * to drain).  NULL is a no-op. */
void moe_ffn_destroy(moe_ffn_plan_t plan);

/* Profiling hooks for the benchmark.  While enabled, every later forward
 * brackets each kernel launch with a pair of timing events on the stream that
 * kernel runs on.  moe_ffn_profile_read waits for the recorded events, adds
 * each kernel's total milliseconds and launch count into the caller's arrays
 * of MOE_FFN_K_COUNT entries (overwriting them), and forgets the records. */
moe_ffn_status moe_ffn_profile_enable(moe_ffn_plan_t plan, int32_t enable);
moe_ffn_status moe_ffn_profile_read(moe_ffn_plan_t plan, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */

// layer_loop -- runs the MoE decode FFN layer through the C ABI alone (no
// Python, no torch): a plain C-ABI usage example and a small driver for
// profiler runs (kernel traces, hardware counters).
//
//   layer_loop <workload> [mode] [steps] [warmup] [launch]
//     workload: decode_bf16_t1 | decode_bf16_t8 | decode_q4_t1_t4 | decode_q4_t1 |
//               decode_bf16_t128 | prefill_bf16_t4096 | prefill_bf16_t16384 |
//               decode_bf16_t1_tp8 | decode_bf16_t8_tp8 | tiny_fp32
//     mode:     auto | aux | seq | fused          (default auto)
//     launch:   eager | graph                     (default eager; graph: one HIP graph
//               captures a rotation window of forwards and is replayed)
//
// Weights and tokens are hash-filled on the device (a fixed seed per layer
// copy); the layers rotate over enough copies that consecutive uses of one
// copy are hundreds of MB apart, as in bench.py.  Prints one line: the
// workload, the shape, the mode and the microseconds per forward (host clock
// around the timed loop, synchronised at both ends).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "moe_ffn.h"

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                 \
        }                                                                                 \
    } while (0)

namespace {

__device__ __forceinline__ uint32_t mix(uint64_t i, uint32_t seed) {
    uint32_t h = (uint32_t)i * 2654435761u ^ (uint32_t)(i >> 32) * 40503u ^ seed * 2246822519u;
    h ^= h >> 15;
    h *= 0x2c1b3c6du;
    h ^= h >> 12;
    h *= 0x297a2d39u;
    h ^= h >> 15;
    return h;
}

// uniform in [-a, a)
__device__ __forceinline__ float unif(uint64_t i, uint32_t seed, float a) {
    return ((mix(i, seed) >> 8) * (1.0f / 16777216.0f) * 2.f - 1.f) * a;
}

__global__ void fill_f32(float *p, size_t n, uint32_t seed, float a) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = unif(i, seed, a);
}

__global__ void fill_bf16(uint16_t *p, size_t n, uint32_t seed, float a) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = __builtin_bit_cast(uint16_t, (__bf16)unif(i, seed, a));
}

__global__ void fill_u8(uint8_t *p, size_t n, uint32_t seed) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = (uint8_t)mix(i, seed);
}

// fp16 block scales in [0.001, 0.01)
__global__ void fill_scale(uint16_t *p, size_t n, uint32_t seed) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = __builtin_bit_cast(uint16_t, (_Float16)(0.0055f + unif(i, seed, 0.0045f)));
}

struct Workload {
    const char *name;
    int H, E, k, I, Is, T;
    int x_dtype, w_dtype;
};

const Workload kWorkloads[] = {
    {"tiny_fp32", 64, 8, 2, 32, 32, 1, MOE_FFN_F32, MOE_FFN_F32},
    {"decode_bf16_t1", 2048, 256, 8, 512, 512, 1, MOE_FFN_BF16, MOE_FFN_BF16},
    {"decode_bf16_t8", 2048, 256, 8, 512, 512, 8, MOE_FFN_BF16, MOE_FFN_BF16},
    {"decode_q4_t1_t4", 2048, 256, 8, 512, 512, 4, MOE_FFN_BF16, MOE_FFN_Q4_B32},
    {"decode_q4_t1", 2048, 256, 8, 512, 512, 1, MOE_FFN_BF16, MOE_FFN_Q4_B32},
    {"decode_bf16_t128", 2048, 256, 8, 512, 512, 128, MOE_FFN_BF16, MOE_FFN_BF16},
    {"prefill_bf16_t4096", 2048, 256, 8, 512, 512, 4096, MOE_FFN_BF16, MOE_FFN_BF16},
    {"prefill_bf16_t16384", 2048, 256, 8, 512, 512, 16384, MOE_FFN_BF16, MOE_FFN_BF16},
    // one GPU's shard of the layer split eight ways inside every expert
    {"decode_bf16_t1_tp8", 2048, 256, 8, 64, 64, 1, MOE_FFN_BF16, MOE_FFN_BF16},
    {"decode_bf16_t8_tp8", 2048, 256, 8, 64, 64, 8, MOE_FFN_BF16, MOE_FFN_BF16},
};

size_t elem_bytes(int dtype) { return dtype == MOE_FFN_F32 ? 4 : 2; }

// bytes of a [rows, K] matrix in the given storage (4-bit: half a byte per weight)
size_t mat_bytes(int dtype, size_t rows, size_t K) {
    return dtype == MOE_FFN_Q4_B32 ? rows * K / 2 : rows * K * elem_bytes(dtype);
}

void *dalloc(size_t n) {
    void *p = nullptr;
    CHECK(hipMalloc(&p, n < 16 ? 16 : n));
    return p;
}

// fills a weight matrix (and, for 4-bit storage, its scales)
void fill_weights(int dtype, void *w, void **scale, size_t rows, size_t K, uint32_t seed) {
    const dim3 g(1024), b(256);
    if (dtype == MOE_FFN_F32) {
        hipLaunchKernelGGL(fill_f32, g, b, 0, 0, (float *)w, rows * K, seed, 0.035f);
    } else if (dtype == MOE_FFN_BF16) {
        hipLaunchKernelGGL(fill_bf16, g, b, 0, 0, (uint16_t *)w, rows * K, seed, 0.035f);
    } else {
        hipLaunchKernelGGL(fill_u8, g, b, 0, 0, (uint8_t *)w, rows * K / 2, seed);
        *scale = dalloc(rows * (K / 32) * 2);
        hipLaunchKernelGGL(fill_scale, g, b, 0, 0, (uint16_t *)*scale, rows * (K / 32), seed ^ 0x5bd1e995u);
    }
    CHECK(hipGetLastError());
}

}  // namespace

int main(int argc, char **argv) {
    if (argc < 2) {
        std::fprintf(stderr, "usage: layer_loop <workload> [auto|aux|seq|fused] [steps] [warmup]\n");
        return 2;
    }
    const Workload *wl = nullptr;
    for (const Workload &w : kWorkloads)
        if (std::strcmp(argv[1], w.name) == 0) wl = &w;
    if (!wl) {
        std::fprintf(stderr, "unknown workload %s\n", argv[1]);
        return 2;
    }
    const std::string mode = argc > 2 ? argv[2] : "auto";
    uint32_t flags = MOE_FFN_SHARED_AUTO;
    if (mode == "aux") flags = MOE_FFN_SHARED_AUX;
    else if (mode == "seq") flags = MOE_FFN_SHARED_SEQ;
    else if (mode == "fused") flags = MOE_FFN_SHARED_FUSED;
    else if (mode != "auto") {
        std::fprintf(stderr, "unknown mode %s\n", mode.c_str());
        return 2;
    }
    const int steps = argc > 3 ? std::atoi(argv[3]) : 2000;
    const int warmup = argc > 4 ? std::atoi(argv[4]) : 200;
    const std::string launch = argc > 5 ? argv[5] : "eager";
    if (launch != "eager" && launch != "graph") {
        std::fprintf(stderr, "unknown launch %s\n", launch.c_str());
        return 2;
    }
    const int H = wl->H, E = wl->E, k = wl->k, I = wl->I, Is = wl->Is, T = wl->T;
    const int wd = wl->w_dtype;

    moe_ffn_desc d{};
    d.hidden = H; d.n_experts = E; d.top_k = k; d.inter = I; d.shared_inter = Is;
    d.max_tokens = T; d.device = 0; d.x_dtype = wl->x_dtype; d.weight_dtype = wd;
    d.flags = flags; d.matvec_max_tokens = 0;
    moe_ffn_plan_t plan = nullptr;
    size_t ws_bytes = 0;
    if (moe_ffn_plan(&d, &plan, &ws_bytes) != MOE_FFN_OK) {
        std::fprintf(stderr, "moe_ffn_plan: %s\n", moe_ffn_last_error());
        return 1;
    }

    // layer copies: enough that one copy's weights leave the 256 MB cache before reuse,
    // even at one token (k routed experts and the shared one per call read 512 MiB
    // between two uses of a copy)
    const size_t layer_bytes = mat_bytes(wd, (size_t)E * I, H) * 3 + mat_bytes(wd, Is, H) * 3;
    const size_t expert_bytes = mat_bytes(wd, I, H) * 3 + (wd == MOE_FFN_Q4_B32 ? (size_t)I * H / 32 * 2 * 3 : 0);
    const size_t min_call = (size_t)(k + 1) * expert_bytes;
    const int base = wd == MOE_FFN_Q4_B32 ? 32 : 16;
    const int rot = (int)std::min<size_t>(128, (((size_t)512 << 20) + min_call - 1) / min_call + 1);
    const int copies = layer_bytes > ((size_t)64 << 20) ? std::max(base, rot) : 2;
    std::vector<moe_ffn_tensors> ts(copies);
    void *x = dalloc((size_t)T * H * elem_bytes(wl->x_dtype));
    float *out = (float *)dalloc((size_t)T * H * 4);
    void *ws = dalloc(ws_bytes);
    if (wl->x_dtype == MOE_FFN_F32)
        hipLaunchKernelGGL(fill_f32, dim3(64), dim3(256), 0, 0, (float *)x, (size_t)T * H, 7u, 1.7f);
    else
        hipLaunchKernelGGL(fill_bf16, dim3(64), dim3(256), 0, 0, (uint16_t *)x, (size_t)T * H, 7u, 1.7f);
    for (int c = 0; c < copies; ++c) {
        moe_ffn_tensors &t = ts[c];
        std::memset(&t, 0, sizeof t);
        const uint32_t s = 100u + 16u * (uint32_t)c;
        float *router = (float *)dalloc((size_t)E * H * 4);
        float *gvec = (float *)dalloc((size_t)H * 4);
        hipLaunchKernelGGL(fill_f32, dim3(256), dim3(256), 0, 0, router, (size_t)E * H, s, 0.035f);
        hipLaunchKernelGGL(fill_f32, dim3(8), dim3(256), 0, 0, gvec, (size_t)H, s + 1, 0.035f);
        void *g = dalloc(mat_bytes(wd, (size_t)E * I, H)), *u = dalloc(mat_bytes(wd, (size_t)E * I, H));
        void *dn = dalloc(mat_bytes(wd, (size_t)E * H, I));
        void *sg = dalloc(mat_bytes(wd, Is, H)), *su = dalloc(mat_bytes(wd, Is, H));
        void *sd = dalloc(mat_bytes(wd, H, Is));
        void *gs = nullptr, *us = nullptr, *ds = nullptr, *sgs = nullptr, *sus = nullptr, *sds = nullptr;
        fill_weights(wd, g, &gs, (size_t)E * I, H, s + 2);
        fill_weights(wd, u, &us, (size_t)E * I, H, s + 3);
        fill_weights(wd, dn, &ds, (size_t)E * H, I, s + 4);
        fill_weights(wd, sg, &sgs, Is, H, s + 5);
        fill_weights(wd, su, &sus, Is, H, s + 6);
        fill_weights(wd, sd, &sds, H, Is, s + 7);
        t.x = x; t.w_router = router; t.gate_vec = gvec; t.out = out;
        t.w_gate = g; t.w_up = u; t.w_down = dn; t.sh_gate = sg; t.sh_up = su; t.sh_down = sd;
        t.w_gate_scale = (const uint16_t *)gs; t.w_up_scale = (const uint16_t *)us;
        t.w_down_scale = (const uint16_t *)ds; t.sh_gate_scale = (const uint16_t *)sgs;
        t.sh_up_scale = (const uint16_t *)sus; t.sh_down_scale = (const uint16_t *)sds;
    }
    CHECK(hipDeviceSynchronize());

    hipStream_t stream;
    CHECK(hipStreamCreate(&stream));
    auto run = [&](int n, int from) {
        for (int i = 0; i < n; ++i) {
            const moe_ffn_status st = moe_ffn_forward(plan, &ts[(from + i) % copies], T, ws, ws_bytes, stream);
            if (st != MOE_FFN_OK) {
                std::fprintf(stderr, "moe_ffn_forward: %s\n", moe_ffn_last_error());
                std::exit(1);
            }
        }
    };
    // graph mode: the first forward (the plan's set-up) runs eagerly, then one graph holds a
    // window of forwards over every layer copy and is replayed
    hipGraphExec_t exec = nullptr;
    hipGraph_t graph = nullptr;
    if (launch == "graph") {
        run(1, 0);
        CHECK(hipStreamSynchronize(stream));
        CHECK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
        run(copies, 0);
        CHECK(hipStreamEndCapture(stream, &graph));
        CHECK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
    }
    auto go = [&](int n, int from) {
        if (launch == "eager") {
            run(n, from);
            return;
        }
        for (int i = 0; i < (n + copies - 1) / copies; ++i) CHECK(hipGraphLaunch(exec, stream));
    };
    const int done = launch == "graph" ? (steps + copies - 1) / copies * copies : steps;
    go(warmup, 0);
    CHECK(hipStreamSynchronize(stream));
    const auto t0 = std::chrono::steady_clock::now();
    go(steps, warmup);
    CHECK(hipStreamSynchronize(stream));
    const double us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
    std::printf("layer_loop %s H=%d E=%d k=%d I=%d Is=%d T=%d mode=%s launch=%s copies=%d steps=%d: %.3f us/forward\n",
                wl->name, H, E, k, I, Is, T, mode.c_str(), launch.c_str(), copies, done, us / done);
    if (exec) CHECK(hipGraphExecDestroy(exec));
    if (graph) CHECK(hipGraphDestroy(graph));
    moe_ffn_destroy(plan);
    CHECK(hipStreamDestroy(stream));
    return 0;
}

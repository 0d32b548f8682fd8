// grid_barrier -- what a grid-wide barrier costs on this GPU, the price of
// turning the layer's kernel boundaries into phases of one persistent kernel.
//
//   grid_barrier <workgroups> [launches]
//
// Each launch: every workgroup (256 threads) writes 1 KiB, crosses a barrier,
// and reads the 1 KiB another workgroup wrote (half the grid away, so on
// another XCD under the round-robin dispatch the driver also checks).  Four
// kernels, timed with events around `launches` back-to-back launches each:
//   plain none   an ordinary launch with no barrier (the floor of a kernel boundary)
//   coop  none   the same kernel, cooperative launch (what guarantees co-residency)
//   coop  flat   every workgroup: agent-scope release fence, one shared counter,
//                spin, agent-scope acquire fence
//   coop  xcd    per-XCD counters (the hardware XCC id); only the last workgroup
//                of each XCD fences and counts in globally; every workgroup then
//                acquires with an agent-scope fence
//   coop  xcd-c  as xcd, but the readers use agent-scope (coherent) loads for the
//                exchanged data instead of the acquire fence
// Spins are bounded (a timeout is counted and reported, never a hang), and the
// values read back are checked.  The kernel trace of a profiler run over this
// driver gives the barrier cost without the host-side launch cost.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                 \
        }                                                                                 \
    } while (0)

namespace {

constexpr unsigned kSpinLimit = 1u << 14;
constexpr int kThreads = 256;
enum Variant { NONE = 0, FLAT = 1, XCD = 2, XCD_COHERENT = 3 };

__device__ __forceinline__ unsigned xcc_id() {
    unsigned v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return v & 15;
}

// ctr: [0] global counter, [16 + 16 x] the counter of XCD x; err: [0] wrong values, [1] spin timeouts
template <int V>
__global__ __launch_bounds__(kThreads) void k_barrier(float *data, unsigned *ctr, unsigned *err,
                                                      unsigned *xcc, unsigned epoch, int per_xcd) {
    const int b = blockIdx.x, G = gridDim.x, tid = threadIdx.x;
    const float mine = (float)(b * 1000 + tid) + (float)epoch * 0.5f;
    data[(size_t)b * kThreads + tid] = mine;
    const unsigned x = xcc_id();
    if (tid == 0 && epoch == 1) xcc[b] = x;
    if (V == FLAT) {
        __syncthreads();
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            unsigned n = 0;
            while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < epoch * (unsigned)G &&
                   ++n < kSpinLimit)
                __builtin_amdgcn_s_sleep(1);
            if (n >= kSpinLimit) atomicAdd(err + 1, 1u);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
    } else if (V == XCD || V == XCD_COHERENT) {
        __syncthreads();
        if (tid == 0) {
            __builtin_amdgcn_s_waitcnt(0);  // this workgroup's stores have reached its L2
            const unsigned old = __hip_atomic_fetch_add(ctr + 16 + 16 * x, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == epoch * (unsigned)per_xcd) {  // the XCD's last: publish its L2, count in
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            unsigned n = 0;
            while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < epoch * 8u &&
                   ++n < kSpinLimit)
                __builtin_amdgcn_s_sleep(1);
            if (n >= kSpinLimit) atomicAdd(err + 1, 1u);
            if (V == XCD) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
    }
    const int o = (b + G / 2 + 1) % G;
    const float want = (float)(o * 1000 + tid) + (float)epoch * 0.5f;
    float v;
    if (V == XCD_COHERENT)
        v = __hip_atomic_load(data + (size_t)o * kThreads + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        v = data[(size_t)o * kThreads + tid];
    if (V != NONE && v != want) atomicAdd(err, 1u);
}

template <int V>
void run(const char *name, bool coop, int G, int launches, float *data, unsigned *ctr, unsigned *err,
         unsigned *xcc, hipStream_t s) {
    CHECK(hipMemset(ctr, 0, 1024 * sizeof(unsigned)));
    CHECK(hipMemset(err, 0, 2 * sizeof(unsigned)));
    CHECK(hipDeviceSynchronize());
    int per_xcd = G / 8;
    hipEvent_t a, z;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&z));
    const int warm = 20;
    for (int i = 0; i < launches + warm; ++i) {
        if (i == warm) CHECK(hipEventRecord(a, s));
        unsigned epoch = (unsigned)i + 1;
        if (coop) {
            void *args[] = {&data, &ctr, &err, &xcc, &epoch, &per_xcd};
            CHECK(hipLaunchCooperativeKernel((const void *)k_barrier<V>, dim3(G), dim3(kThreads), args, 0, s));
        } else {
            hipLaunchKernelGGL(k_barrier<V>, dim3(G), dim3(kThreads), 0, s, data, ctr, err, xcc, epoch, per_xcd);
            CHECK(hipGetLastError());
        }
    }
    CHECK(hipEventRecord(z, s));
    CHECK(hipEventSynchronize(z));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, a, z));
    unsigned h[2];
    CHECK(hipMemcpy(h, err, sizeof h, hipMemcpyDeviceToHost));
    std::printf("%-5s %-6s G=%d: %8.3f us per launch (host clock of %d launches)  wrong_values=%u spin_timeouts=%u\n",
                coop ? "coop" : "plain", name, G, ms * 1000.0 / launches, launches, h[0], h[1]);
    std::fflush(stdout);
    CHECK(hipEventDestroy(a));
    CHECK(hipEventDestroy(z));
}

}  // namespace

int main(int argc, char **argv) {
    if (argc < 2) {
        std::fprintf(stderr, "usage: grid_barrier <workgroups: multiple of 8> [launches]\n");
        return 2;
    }
    const int G = std::atoi(argv[1]);
    const int launches = argc > 2 ? std::atoi(argv[2]) : 2000;
    int occ = 0, cus = 0;
    CHECK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_barrier<FLAT>, kThreads, 0));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    if (G <= 0 || G % 8 != 0 || G > occ * cus || G > 1024 || launches <= 0) {
        std::fprintf(stderr, "workgroups must be a multiple of 8, at most %d (co-resident) and 1024\n",
                     occ * cus < 1024 ? occ * cus : 1024);
        return 2;
    }
    float *data;
    unsigned *ctr, *err, *xcc;
    CHECK(hipMalloc(&data, (size_t)G * kThreads * sizeof(float)));
    CHECK(hipMalloc(&ctr, 1024 * sizeof(unsigned)));
    CHECK(hipMalloc(&err, 2 * sizeof(unsigned)));
    CHECK(hipMalloc(&xcc, (size_t)G * sizeof(unsigned)));
    hipStream_t s;
    CHECK(hipStreamCreate(&s));
    std::printf("grid_barrier: %d workgroups of %d threads, %d resident per CU, %d CUs\n", G, kThreads, occ, cus);
    run<NONE>("none", false, G, launches, data, ctr, err, xcc, s);
    run<NONE>("none", true, G, launches, data, ctr, err, xcc, s);
    run<FLAT>("flat", true, G, launches, data, ctr, err, xcc, s);
    run<XCD>("xcd", true, G, launches, data, ctr, err, xcc, s);
    run<XCD_COHERENT>("xcd-c", true, G, launches, data, ctr, err, xcc, s);
    std::vector<unsigned> h(G);
    CHECK(hipMemcpy(h.data(), xcc, (size_t)G * sizeof(unsigned), hipMemcpyDeviceToHost));
    int count[16] = {0}, round_robin = 1;
    for (int i = 0; i < G; ++i) {
        count[h[i] & 15]++;
        if ((int)(h[i] & 15) != i % 8) round_robin = 0;
    }
    std::printf("workgroups per XCD:");
    for (int i = 0; i < 8; ++i) std::printf(" %d", count[i]);
    std::printf("  (round-robin by workgroup id: %s)\n", round_robin ? "yes" : "no");
    CHECK(hipStreamDestroy(s));
    return 0;
}

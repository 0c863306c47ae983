// stream_ceiling.hip - streaming-ceiling kernels for gfx950 (measurement only;
// C ABI in stream_ceiling.h). Each call reads NI buffers and writes NO buffers
// of the same size once, in the access pattern of the all-reduce sum kernel
// (512 lanes x 2 packs of 16 bytes per step, non-temporal), with no other work.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "stream_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kUnroll = 2;
constexpr unsigned kMaxGrid = 1u << 20;

struct StreamArgs {
    const u32x4 *in[SC_MAX_IN];
    u32x4 *out[SC_MAX_OUT];
    size_t npacks;
};

template <int NI, int NO>
__device__ __forceinline__ void one_pack(const StreamArgs &a, size_t j)
{
    u32x4 x = __builtin_nontemporal_load(a.in[0] + j);
#pragma unroll
    for (int r = 1; r < NI; ++r)
        x ^= __builtin_nontemporal_load(a.in[r] + j);
#pragma unroll
    for (int k = 0; k < NO; ++k)
        __builtin_nontemporal_store(x, a.out[k] + j);
    if (NO == 0)
        asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}

template <int NI, int NO>
__global__ __launch_bounds__(kThreads) void stream_kernel(StreamArgs a)
{
    const size_t step = static_cast<size_t>(kThreads) * kUnroll;
    const size_t nfull = a.npacks / step;
    for (size_t c = blockIdx.x; c < nfull; c += gridDim.x) {
        const size_t base = c * step + threadIdx.x;
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            x[u] = __builtin_nontemporal_load(a.in[0] + base + u * kThreads);
#pragma unroll
        for (int r = 1; r < NI; ++r)
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                x[u] ^= __builtin_nontemporal_load(a.in[r] + base + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < NO; ++k)
                __builtin_nontemporal_store(x[u], a.out[k] + base + u * kThreads);
            if (NO == 0)
                asm volatile("" ::"v"(x[u].x), "v"(x[u].y), "v"(x[u].z), "v"(x[u].w));
        }
    }
    if (blockIdx.x == gridDim.x - 1)
        for (size_t j = nfull * step + threadIdx.x; j < a.npacks; j += kThreads)
            one_pack<NI, NO>(a, j);
}

template <int NI, int NO>
int32_t launch(const StreamArgs &a, hipStream_t stream)
{
    size_t blocks = a.npacks / (static_cast<size_t>(kThreads) * kUnroll);
    const unsigned grid = blocks < 1 ? 1u : blocks > kMaxGrid ? kMaxGrid : static_cast<unsigned>(blocks);
    hipLaunchKernelGGL((stream_kernel<NI, NO>), dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? SC_OK : SC_ERR_HIP;
}

template <int NO>
int32_t by_inputs(int n_in, const StreamArgs &a, hipStream_t s)
{
    switch (n_in) {
    case 1: return launch<1, NO>(a, s);
    case 2: return launch<2, NO>(a, s);
    case 3: return launch<3, NO>(a, s);
    case 4: return launch<4, NO>(a, s);
    case 5: return launch<5, NO>(a, s);
    case 6: return launch<6, NO>(a, s);
    case 7: return launch<7, NO>(a, s);
    case 8: return launch<8, NO>(a, s);
    case 9: return launch<9, NO>(a, s);
    case 10: return launch<10, NO>(a, s);
    case 11: return launch<11, NO>(a, s);
    default: return launch<12, NO>(a, s);
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int32_t sc_stream(const void *const *in, int32_t n_in, void *const *out, int32_t n_out, size_t bytes,
                             void *hip_stream)
{
    if (n_in < 1 || n_in > SC_MAX_IN || n_out < 0 || n_out > SC_MAX_OUT)
        return SC_ERR_COUNT;
    if (!in || (n_out > 0 && !out))
        return SC_ERR_NULL;
    if (bytes % 16 != 0)
        return SC_ERR_ALIGN;
    StreamArgs a = {};
    for (int r = 0; r < n_in; ++r) {
        if (!in[r])
            return SC_ERR_NULL;
        if (!aligned16(in[r]))
            return SC_ERR_ALIGN;
        a.in[r] = static_cast<const u32x4 *>(in[r]);
    }
    for (int k = 0; k < n_out; ++k) {
        if (!out[k])
            return SC_ERR_NULL;
        if (!aligned16(out[k]))
            return SC_ERR_ALIGN;
        a.out[k] = static_cast<u32x4 *>(out[k]);
    }
    a.npacks = bytes / 16;
    if (a.npacks == 0)
        return SC_OK;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    switch (n_out) {
    case 0: return by_inputs<0>(n_in, a, s);
    case 1: return by_inputs<1>(n_in, a, s);
    default: return by_inputs<2>(n_in, a, s);
    }
}

// stream_ceiling.hip - streaming-ceiling kernels for gfx950 (measurement only;
// C ABI in stream_ceiling.h). Each call reads NI buffers and writes NO buffers
// of the same size once, with no other work, in one of a few workgroup shapes
// (lanes x packs per lane per step), one of two load forms and one of two
// store forms. Loads are 16-byte and non-temporal: global loads from 64-bit
// per-lane addresses, or buffer loads from the step's start address (a
// workgroup-uniform resource and a 32-bit lane offset, which leaves far more
// registers free and so more waves resident). Stores are non-temporal global
// stores, or buffer stores at device scope (cache-policy field sc1) from the
// step's start address. No single variant is fastest for every mix of
// streams, so a caller times each.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "stream_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

constexpr int kBufferWord3 = 0x00020000;  // raw (untyped) 32-bit data format
constexpr int kPolicySc1 = 16;            // cache-policy field: sc1 (device scope), temporal
constexpr int kPolicyNt = 2;              // cache-policy field: nt (non-temporal)

// Pack at byte offset `off` of the `extent` bytes from `base` (the same in
// every lane of the wave), non-temporal.
__device__ __forceinline__ u32x4 load_buf(const u32x4 *base, uint32_t off, uint32_t extent)
{
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(base), 0, static_cast<int>(extent), kBufferWord3);
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kPolicyNt);
}

// Pack at byte offset `off` of the `extent` bytes from `base`; `base` is the
// same in every lane of the wave.
__device__ __forceinline__ void store_sc1(u32x4 *base, uint32_t off, uint32_t extent, u32x4 v)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(extent), kBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, kPolicySc1);
}

// Pack `base + u * kThreads` of input r in a full step that starts at pack
// `c * step`: a global load, or (BL) a buffer load from the step's start.
template <int kThreads, bool BL>
__device__ __forceinline__ u32x4 step_load(const u32x4 *in, size_t c, size_t step, size_t base, int u)
{
    if (BL)
        return load_buf(in + c * step, (threadIdx.x + u * kThreads) * 16u, static_cast<uint32_t>(step * 16u));
    return __builtin_nontemporal_load(in + base + u * kThreads);
}

// kThreads lanes x kUnroll packs per step; consecutive steps go to
// consecutive workgroups; the packs after the last full step are done by the
// last workgroup. SC1: the full steps' stores are device-scope buffer stores;
// BL: the full steps' loads are buffer loads.
template <int NI, int NO, int kThreads, int kUnroll, bool SC1, bool BL>
__global__ __launch_bounds__(kThreads) void stream_kernel(StreamArgs a)
{
    const size_t step = static_cast<size_t>(kThreads) * kUnroll;
    const size_t nfull = a.npacks / step;
    for (size_t c = blockIdx.x; c < nfull; c += gridDim.x) {
        const size_t base = c * step + threadIdx.x;
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            x[u] = step_load<kThreads, BL>(a.in[0], c, step, base, u);
#pragma unroll
        for (int r = 1; r < NI; ++r)
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                x[u] ^= step_load<kThreads, BL>(a.in[r], c, step, base, u);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < NO; ++k) {
                if (SC1)
                    store_sc1(a.out[k] + c * step, (threadIdx.x + u * kThreads) * 16u, step * 16u, x[u]);
                else
                    __builtin_nontemporal_store(x[u], a.out[k] + base + u * kThreads);
            }
            if (NO == 0)
                asm volatile("" ::"v"(x[u].x), "v"(x[u].y), "v"(x[u].z), "v"(x[u].w));
        }
    }
    if (blockIdx.x == gridDim.x - 1)
        for (size_t j = nfull * step + threadIdx.x; j < a.npacks; j += kThreads)
            one_pack<NI, NO>(a, j);
}

template <int NI, int NO, int T, int U, bool SC1, bool BL>
int32_t launch(const StreamArgs &a, hipStream_t stream)
{
    size_t blocks = a.npacks / (static_cast<size_t>(T) * U);
    const unsigned grid = blocks < 1 ? 1u : blocks > kMaxGrid ? kMaxGrid : static_cast<unsigned>(blocks);
    hipLaunchKernelGGL((stream_kernel<NI, NO, T, U, SC1, BL>), dim3(grid), dim3(T), 0, stream, a);
    return hipGetLastError() == hipSuccess ? SC_OK : SC_ERR_HIP;
}

// Shapes 0-3: the workgroup geometry; + SC_SHAPE_SC1: sc1 buffer stores;
// + SC_SHAPE_BL: buffer loads.
template <int NI, int NO, bool SC1, bool BL>
int32_t by_geometry(int geometry, const StreamArgs &a, hipStream_t s)
{
    switch (geometry) {
    case SC_SHAPE_512x2: return launch<NI, NO, 512, 2, SC1, BL>(a, s);
    case SC_SHAPE_256x4: return launch<NI, NO, 256, 4, SC1, BL>(a, s);
    case SC_SHAPE_256x8: return launch<NI, NO, 256, 8, SC1, BL>(a, s);
    default: return launch<NI, NO, 128, 8, SC1, BL>(a, s);
    }
}

template <int NI, int NO>
int32_t by_shape(int shape, const StreamArgs &a, hipStream_t s)
{
    const int geometry = shape & (SC_SHAPE_SC1 - 1);  // the low bits: SC_SHAPE_512x2 .. SC_SHAPE_128x8
    const bool sc1 = shape & SC_SHAPE_SC1, bl = shape & SC_SHAPE_BL;
    if (bl)
        return sc1 ? by_geometry<NI, NO, true, true>(geometry, a, s) : by_geometry<NI, NO, false, true>(geometry, a, s);
    return sc1 ? by_geometry<NI, NO, true, false>(geometry, a, s) : by_geometry<NI, NO, false, false>(geometry, a, s);
}

template <int NO>
int32_t by_inputs(int n_in, int shape, const StreamArgs &a, hipStream_t s)
{
    switch (n_in) {
    case 1: return by_shape<1, NO>(shape, a, s);
    case 2: return by_shape<2, NO>(shape, a, s);
    case 3: return by_shape<3, NO>(shape, a, s);
    case 4: return by_shape<4, NO>(shape, a, s);
    case 5: return by_shape<5, NO>(shape, a, s);
    case 6: return by_shape<6, NO>(shape, a, s);
    case 7: return by_shape<7, NO>(shape, a, s);
    case 8: return by_shape<8, NO>(shape, a, s);
    case 9: return by_shape<9, NO>(shape, a, s);
    case 10: return by_shape<10, NO>(shape, a, s);
    case 11: return by_shape<11, NO>(shape, a, s);
    default: return by_shape<12, NO>(shape, a, s);
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int32_t sc_stream(const void *const *in, int32_t n_in, void *const *out, int32_t n_out, size_t bytes,
                             int32_t shape, void *hip_stream)
{
    if (n_in < 1 || n_in > SC_MAX_IN || n_out < 0 || n_out > SC_MAX_OUT)
        return SC_ERR_COUNT;
    if (shape < 0 || shape >= SC_NUM_SHAPES)
        return SC_ERR_SHAPE;
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
    case 0: return by_inputs<0>(n_in, shape, a, s);
    case 1: return by_inputs<1>(n_in, shape, a, s);
    default: return by_inputs<2>(n_in, shape, a, s);
    }
}

// Measurement utility, not a step of the decode: a plain streaming read of a
// device buffer with the same 16-byte non-temporal loads the heads use. It
// gives the attainable HBM read bandwidth on the running GPU and a kernel of
// exactly known traffic for scaling hardware byte counters.
#include "md_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int BLOCK = 256;
constexpr int UNROLL = 16;

// Each wave streams its own contiguous range, 16 loads deep (on MI355X this
// reads faster than a grid-stride loop, whose consecutive loads of a wave lie
// megabytes apart).
__global__ __launch_bounds__(BLOCK) void k_stream_read(const u32x4* __restrict__ p, size_t n16, unsigned* __restrict__ sink) {
    const size_t nw = (size_t)gridDim.x * (BLOCK / 64);
    const size_t wid = (size_t)blockIdx.x * (BLOCK / 64) + threadIdx.x / 64;
    const size_t end = n16 * (wid + 1) / nw;
    const size_t stride = 64;
    unsigned acc = 0;
    size_t i = n16 * wid / nw + (threadIdx.x & 63);
    n16 = end;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // keep the loads live: one word per block
    __shared__ unsigned s[BLOCK];
    s[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned a = 0;
        for (int t = 0; t < BLOCK; ++t) a ^= s[t];
        sink[blockIdx.x] = a;
    }
}

}  // namespace

int probe_blocks() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                   hipSuccess || n <= 0)
        n = 256;
    return 2 * n;
}

hipError_t probe_launch(const void* buf, size_t bytes, void* sink, hipStream_t s) {
    hipLaunchKernelGGL(k_stream_read, dim3(probe_blocks()), dim3(BLOCK), 0, s, reinterpret_cast<const u32x4*>(buf),
                       bytes / 16, reinterpret_cast<unsigned*>(sink));
    return hipGetLastError();
}

// Measurement helper: the achievable HBM read rate.  A grid-stride stream of
// 128-bit non-temporal loads (the load the GEMV uses for its weights), four
// in flight per thread, folded by XOR into one word per workgroup so that no
// load is dead.  It computes nothing of the method; the roofline of the
// streaming kernels is reported against its rate next to the chip's peak.
#include "internal.h"

namespace qk {

namespace {

typedef unsigned pv4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold_nt(const uint4* p) {
    const pv4u v = __builtin_nontemporal_load(reinterpret_cast<const pv4u*>(p));
    return v.x ^ v.y ^ v.z ^ v.w;
}

__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ p, uint64_t n16,
                                                    uint32_t* __restrict__ out) {
    __shared__ uint32_t red[4];
    constexpr uint64_t CH = 4 * 256;   // 16-byte words per workgroup per step
    const uint64_t stride = (uint64_t)gridDim.x * CH;
    uint32_t acc = 0;
    uint64_t i = (uint64_t)blockIdx.x * CH + threadIdx.x;
    for (; i + 3 * 256 < n16; i += stride)   // whole steps: four loads issued together
        acc ^= fold_nt(p + i) ^ fold_nt(p + i + 256) ^ fold_nt(p + i + 512) ^ fold_nt(p + i + 768);
    for (; i < n16; i += 256) acc ^= fold_nt(p + i);   // the ragged last step
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, WAVE);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

}  // namespace qk

using namespace qk;

extern "C" int qk_read_probe(const void* buf, int64_t bytes, uint32_t* out, int32_t blocks,
                             void* stream) {
    QK_REQUIRE(bytes >= 0 && blocks > 0 && blocks <= 65536, QK_EINVAL);
    QK_REQUIRE(bytes % 16 == 0, QK_ESHAPE);
    QK_REQUIRE(buf && out, QK_EINVAL);
    QK_REQUIRE(QK_ALIGNED(buf, 16) && QK_ALIGNED(out, 4), QK_EALIGN);
    hipLaunchKernelGGL(k_read_probe, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(buf), (uint64_t)bytes / 16u, out);
    return qk_launch_status();
}

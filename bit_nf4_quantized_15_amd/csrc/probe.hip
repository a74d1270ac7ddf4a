// Plain-read probe: streams a device buffer through registers and writes nothing (a
// store that never happens keeps the loads alive).  A measurement aid, not a step of
// the layer: it gives the bandwidth that a launch reading the same number of bytes
// reaches with no compute, the ceiling next to which the decode forward is reported.
#include "common.h"

namespace qlora {
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// lane g of the grid reads 16-byte chunks g, g + L, ..., g + (PER - 1) L (L = lanes of the grid)
template <int PER>
__global__ __launch_bounds__(512) void read_probe_kernel(const uint8_t* src, uint32_t bytes, uint32_t* sink) {
    const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), (short)0, (int)bytes, 0x00020000);
    const uint32_t lanes = gridDim.x * blockDim.x, g = blockIdx.x * blockDim.x + threadIdx.x;
    u32x4_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)      // chunks past the end read as zeros (range-checked loads)
        v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, 16u * (g + lanes * i), 0, 0));
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if (x == 0x9E3779B9u && g == 0) sink[0] = x;
}

}  // namespace
}  // namespace qlora

extern "C" qlora_status qlora_read_probe(const void* src, size_t bytes, uint32_t* sink, int variant, void* stream) {
    using namespace qlora;
    if (!src || !sink || bytes == 0 || bytes >= (size_t(1) << 31) || (variant != 0 && variant != 1))
        return QLORA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 15u))
        return QLORA_ERR_MISALIGNED;
    const uint32_t chunks = (uint32_t)((bytes + 15) / 16);
    const int threads = variant == 0 ? 256 : 512, per = variant == 0 ? 4 : 8;
    const uint32_t blocks = (chunks + (uint32_t)(threads * per) - 1) / (uint32_t)(threads * per);
    hipStream_t s = (hipStream_t)stream;
    if (variant == 0)
        hipLaunchKernelGGL(read_probe_kernel<4>, dim3(blocks), dim3(threads), 0, s, (const uint8_t*)src,
                           (uint32_t)bytes, sink);
    else
        hipLaunchKernelGGL(read_probe_kernel<8>, dim3(blocks), dim3(threads), 0, s, (const uint8_t*)src,
                           (uint32_t)bytes, sink);
    return hipGetLastError() == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

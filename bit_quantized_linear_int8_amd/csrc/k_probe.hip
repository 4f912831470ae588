// k_probe.hip -- a measurement helper, not part of the method: the HBM read
// stream that bounds one launch of the decode kernel.  A workgroup of 512
// threads reads one contiguous slice of the buffer; each load instruction
// moves lane_bytes per lane (a wave instruction covers 64 * lane_bytes
// contiguous bytes) and U loads per lane are in flight before any is used.
// The data are folded with XOR into a value that is stored only if it equals
// a constant the data never produce, which keeps every load live.
#include "qa_device.hpp"
#include "qa_launch.hpp"

namespace qa {

template <int LB, int U>
__global__ __launch_bounds__(512) void k_stream_read(const uint8_t* __restrict__ src, uint64_t bytes, uint64_t per,
                                                     uint32_t* __restrict__ sink) {
    const uint64_t start = (uint64_t)blockIdx.x * per;
    if (start >= bytes) return;
    const uint64_t len = bytes - start < per ? bytes - start : per;
    const rsrc_t r = make_rsrc(src + start, (int64_t)len);     // loads past the slice read zeros
    constexpr uint32_t STEP = 512u * LB;                          // bytes per load instruction of the block
    uint32_t acc = 0u;
    for (uint64_t base = 0; base < len; base += (uint64_t)STEP * U) {
        uint32_t v[U][LB / 4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t off = (uint32_t)(base + (uint64_t)u * STEP) + threadIdx.x * LB;
            if constexpr (LB == 16) {
                const u32x4 x = bload16(r, off);
                v[u][0] = x[0]; v[u][1] = x[1]; v[u][2] = x[2]; v[u][3] = x[3];
            } else if constexpr (LB == 8) {
                const u32x2 x = bload8(r, off);
                v[u][0] = x[0]; v[u][1] = x[1];
            } else {
                v[u][0] = bload4(r, off);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int d = 0; d < LB / 4; ++d) acc ^= v[u][d];
    }
    if (acc == 0x9e3779b9u) sink[(uint64_t)blockIdx.x * 512 + threadIdx.x] = acc;
}

template <int LB>
static void stream_read_u(int unroll, dim3 grid, hipStream_t st, const uint8_t* src, uint64_t bytes, uint64_t per,
                          uint32_t* sink) {
    switch (unroll) {
        case 1: hipLaunchKernelGGL((k_stream_read<LB, 1>), grid, dim3(512), 0, st, src, bytes, per, sink); break;
        case 2: hipLaunchKernelGGL((k_stream_read<LB, 2>), grid, dim3(512), 0, st, src, bytes, per, sink); break;
        case 4: hipLaunchKernelGGL((k_stream_read<LB, 4>), grid, dim3(512), 0, st, src, bytes, per, sink); break;
        default: hipLaunchKernelGGL((k_stream_read<LB, 8>), grid, dim3(512), 0, st, src, bytes, per, sink); break;
    }
}

hipError_t launch_stream_read(const uint8_t* src, uint64_t bytes, int wgs, int lane_bytes, int unroll, uint32_t* sink,
                              hipStream_t st) {
    // slice per workgroup: a whole number of block-wide load instructions
    const uint64_t step = 512ull * (uint64_t)lane_bytes;
    const uint64_t per = bytes == 0 ? step : ((bytes + (uint64_t)wgs - 1) / (uint64_t)wgs + step - 1) / step * step;
    const dim3 grid((unsigned)wgs);
    if (lane_bytes == 16)
        stream_read_u<16>(unroll, grid, st, src, bytes, per, sink);
    else if (lane_bytes == 8)
        stream_read_u<8>(unroll, grid, st, src, bytes, per, sink);
    else
        stream_read_u<4>(unroll, grid, st, src, bytes, per, sink);
    return hipGetLastError();
}

}  // namespace qa

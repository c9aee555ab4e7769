// The stand-alone sliver kernel: columns past the last full tile of a
// wide output, for the plans whose tiled kernel does not run them itself
// (device code and design in sliver.hpp).
#include "launch.hpp"
#include "sliver.hpp"

namespace dg {

namespace {

template <int AB_TYPE, int NR>
__global__ __launch_bounds__(kSliverThreads) void gemm_sliver_kernel(GemmArgs g, int64_t n0,
                                                                     int32_t nrem)
{
    sliver_block<AB_TYPE, NR>(g, n0, nrem, blockIdx.x, blockIdx.y);
}

template <int AB_TYPE>
hipError_t launch_sliver_t(const GemmArgs &g, int64_t n0, int32_t nrem, hipStream_t stream)
{
    const dim3 grid((unsigned)((g.M + kSliverRowsPerBlock - 1) / kSliverRowsPerBlock),
                    (unsigned)g.sched.batch),
        block(kSliverThreads);
    if (nrem <= 1)
        hipLaunchKernelGGL((gemm_sliver_kernel<AB_TYPE, 1>), grid, block, 0, stream, g, n0, nrem);
    else if (nrem <= 2)
        hipLaunchKernelGGL((gemm_sliver_kernel<AB_TYPE, 2>), grid, block, 0, stream, g, n0, nrem);
    else if (nrem <= 4)
        hipLaunchKernelGGL((gemm_sliver_kernel<AB_TYPE, 4>), grid, block, 0, stream, g, n0, nrem);
    else
        hipLaunchKernelGGL((gemm_sliver_kernel<AB_TYPE, 8>), grid, block, 0, stream, g, n0, nrem);
    return hipGetLastError();
}

} // namespace

hipError_t launch_sliver(const GemmArgs &g, int64_t n0, int32_t nrem, hipStream_t stream)
{
    if (nrem < 1 || nrem > kMaxSliver)
        return hipErrorInvalidValue;
    if (g.ab_type == DT_BF16)
        return launch_sliver_t<DT_BF16>(g, n0, nrem, stream);
    if (g.ab_type == DT_F16)
        return launch_sliver_t<DT_F16>(g, n0, nrem, stream);
    return launch_sliver_t<DT_F32>(g, n0, nrem, stream);
}

} // namespace dg

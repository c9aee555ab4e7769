// Stand-ins for the launchers of the fp32 and 16-bit matrix-core kernel
// families, linked into the host-code sanitizer build of the library
// (tests/test_sanitizers.py) in place of those kernels, whose device code
// takes minutes to compile.  Nothing in that test launches a kernel: every
// call it makes returns during host validation or planning.  Each stand-in
// reports a launch error if it is ever reached.
#include "mfma16.hpp"

namespace dg {

hipError_t launch_mfma16_bf16_a(const GemmArgs &, const Plan &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mfma16_bf16_b(const GemmArgs &, const Plan &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mfma16_f16_a(const GemmArgs &, const Plan &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mfma16_f16_b(const GemmArgs &, const Plan &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mfma16_mn256(const GemmArgs &, const Plan &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mfma16_mn128(const GemmArgs &, const Plan &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mfma_f32(const GemmArgs &, const Plan &, hipStream_t) { return hipErrorInvalidValue; }

} // namespace dg

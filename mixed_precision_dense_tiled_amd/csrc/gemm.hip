// gemm.hip -- host entry of the tiled MFMA GEMMs with the plain epilogue
// (D = A x B + C in the output format): FP16 / BF16 -> FP32 or 16-bit, INT8
// -> INT32; FP8 goes to gemm_fp8_general.hip.  The kernel template and its
// launchers are in gemm_kernel.hpp.
#include "gemm_kernel.hpp"

namespace mpdt {

hipError_t launch_gemm(Kind kind, const GemmArgs& a, bool aligned, hipStream_t stream) {
    switch (kind) {
        case Kind::F16: return launch_mma<Kind::F16, Cfg1W<Kind::F16>, Cfg8W<Kind::F16>>(a, aligned, stream);
        case Kind::BF16:
            return launch_mma<Kind::BF16, Cfg1W<Kind::BF16>, Cfg8W<Kind::BF16>>(a, aligned, stream);
        case Kind::I8: return launch_mma<Kind::I8, Cfg1W<Kind::I8>, Cfg8W<Kind::I8>>(a, aligned, stream);
        case Kind::FP8: return launch_fp8(a, aligned, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mpdt

#ifdef MPDT_CLOCK_STAMPS
// Copy the stamps of the first n workgroups of the last instrumented launch
// (6 per workgroup: shader clock at entry / after the K loop / at the end,
// then the real-time counter at the same three points) to host memory.
extern "C" __attribute__((visibility("default"))) int mpdt_clock_stamps(uint64_t* host, int n) {
    if (n < 0 || n > mpdt::CLOCK_STAMP_WGS) return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(mpdt::g_clock_stamps), (size_t)n * 6 * 8, 0,
                                    hipMemcpyDeviceToHost);
}
#endif

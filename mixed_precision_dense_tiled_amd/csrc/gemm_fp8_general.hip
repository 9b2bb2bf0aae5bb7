// gemm_fp8_general.hip -- host entry of the FP8 GEMMs (block-scaled or
// row-scaled, E4M3 or E5M2 operands, BF16 D): a problem the one-wave kernel
// takes whole (gemm_fp8.hip) goes to it in one launch; where it takes only
// the full tiles, the edge tiles go to the general kernel (gemm_kernel.hpp),
// and so does every other problem; both kernels are instantiated for the
// operand formats and the scaling variant of the call.
#include "gemm_kernel.hpp"

namespace mpdt {

template <int F8>
static hipError_t launch_fp8_t(const GemmArgs& a0, bool aligned, hipStream_t stream) {
    const int mode = fp8_1w_mode(a0, aligned);
    if (mode == 2)
        return launch_fp8_1w(a0, (a0.M + FP8_TILE_M - 1) / FP8_TILE_M, (a0.N + FP8_TILE_N - 1) / FP8_TILE_N,
                             stream);
    const int int_tm = mode ? a0.M / FP8_TILE_M : 0;
    const int int_tn = mode ? a0.N / FP8_TILE_N : 0;
    if (int_tm > 0 && int_tn > 0) {
        const hipError_t e = launch_fp8_1w(a0, int_tm, int_tn, stream);
        if (e != hipSuccess) return e;
        return launch_general<Kind::FP8, CfgFP8, false, F8>(a0, aligned, int_tm, int_tn, stream);
    }
    return launch_general<Kind::FP8, CfgFP8, false, F8>(a0, aligned, 0, 0, stream);
}

hipError_t launch_fp8(const GemmArgs& a, bool aligned, hipStream_t stream) {
    switch (fp8_variant(a)) {
        case 0: return launch_fp8_t<0>(a, aligned, stream);
        case 1: return launch_fp8_t<1>(a, aligned, stream);
        case 2: return launch_fp8_t<2>(a, aligned, stream);
        case 3: return launch_fp8_t<3>(a, aligned, stream);
        case 4: return launch_fp8_t<4>(a, aligned, stream);
        case 5: return launch_fp8_t<5>(a, aligned, stream);
        case 6: return launch_fp8_t<6>(a, aligned, stream);
        case 7: return launch_fp8_t<7>(a, aligned, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mpdt

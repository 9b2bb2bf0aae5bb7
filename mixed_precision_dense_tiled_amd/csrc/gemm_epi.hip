// gemm_epi.hip -- host entry of the FP16 / BF16 MFMA GEMMs with the fused
// epilogue: D = act(A x B + C + bias) in FP32 or in the input format.  The
// bias (one FP32 value per output column) belongs in the floating-point
// epilogue of a linear layer ("NVIDIA A100: from chip to SIMT", section 5.1);
// fusing it and the activation into the GEMM's own epilogue spares the extra
// pass over D that a separate kernel would make.  Same kernel template and
// tile configurations as gemm.hip (gemm_kernel.hpp), instantiated with the
// fused epilogue, in a translation unit of its own so the two build in
// parallel.
#include "gemm_kernel.hpp"

namespace mpdt {

hipError_t launch_gemm_epi(Kind kind, const GemmArgs& a, bool aligned, hipStream_t stream) {
    switch (kind) {
        case Kind::F16:
            return launch_mma<Kind::F16, Cfg1W<Kind::F16>, Cfg8W<Kind::F16>, true>(a, aligned, stream);
        case Kind::BF16:
            return launch_mma<Kind::BF16, Cfg1W<Kind::BF16>, Cfg8W<Kind::BF16>, true>(a, aligned, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mpdt

// gemm_mfma.hip -- bf16 MFMA grouped dequant-GEMMs for gfx950 (filled in below).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace moeq {

hipError_t launch_fast_swiglu(const ProjProblem &p, hipStream_t s, bool *handled) {
    (void)p;
    (void)s;
    *handled = false;
    return hipSuccess;
}

hipError_t launch_fast_plain(const ProjProblem &p, hipStream_t s, bool *handled) {
    (void)p;
    (void)s;
    *handled = false;
    return hipSuccess;
}

}  // namespace moeq

// matmul_grouped16_acc.hip -- the 16x16x1 Grouped kernel (grouped16_kernel.hpp)
// built with its matrix-core accumulators in the accumulation registers,
// for jobs of at most kG16AccRounds rounds of k.
#include "grouped16_kernel.hpp"

namespace eidm {

hipError_t launch_grouped16_acc(const MatmulArgs& a, const MapBuffers& buf, int device_cus,
                                hipStream_t stream) {
    return g16_launch(a, buf, device_cus, stream);
}

}  // namespace eidm

// matmul_grouped16.hip -- Grouped form of the expert-ID matmul for 16-bit
// weights on the 16x16x1 f32 matrix-core step (the kernel and its design:
// grouped16_kernel.hpp).
//
// This source is built with the matrix-core accumulators in the
// architectural registers, where the slice sums at the end of a job are
// read by ordinary adds.  Short jobs (few rounds of k) spend more of their
// time at job boundaries and go to matmul_grouped16_acc.hip, built with
// the accumulators in the accumulation registers: there the rounds leave
// more architectural registers free, at the cost of one move per slice sum
// per job.
#include "grouped16_kernel.hpp"

namespace eidm {

// The kernel needs 16-byte rows (vector loads), at least three rounds, input,
// output and each expert's matrix addressable with 32-bit byte offsets, and
// 16-bit weights.
bool grouped16_supported(const MatmulArgs& a) {
    if (a.dtype != kDtypeF16 && a.dtype != kDtypeBF16) return false;
    if (!a.vec) return false;
    const uint32_t rounds = (a.k + kRoundK - 1) / kRoundK;
    if (rounds < 3) return false;
    const uint64_t routed = (uint64_t)a.m * a.top_k;
    const uint64_t in_rows = a.layout == 1 ? routed : a.m;
    if (in_rows * a.k * 4ull >= 0xffffff00ull) return false;
    if ((uint64_t)a.n * a.k * 2ull + 256 >= 0xffffffffull) return false;
    if (routed * a.n >= 0xffffff00ull) return false;
    return true;
}

hipError_t launch_grouped16(const MatmulArgs& a, const MapBuffers& buf, int device_cus, hipStream_t stream) {
    const uint32_t rounds = (a.k + kRoundK - 1) / kRoundK;
    if (rounds <= kG16AccRounds) return launch_grouped16_acc(a, buf, device_cus, stream);
    return g16_launch(a, buf, device_cus, stream);
}

}  // namespace eidm

// Stand-ins for the kernel launchers of libsgemm, for the host-only
// sanitizer build of the C ABI layer (csrc/sgemm_api.hip): the argument
// validation under test never reaches them; a call that passes validation
// gets hipErrorInvalidDevice back (no GPU is used).
#include "tiles.h"

namespace sgemm {
hipError_t launch_mfma(const GemmArgs&, hipStream_t) { return hipErrorInvalidDevice; }
hipError_t launch_valu(const GemmArgs&, hipStream_t) { return hipErrorInvalidDevice; }
hipError_t launch_valu_page(const GemmArgs&, hipStream_t) { return hipErrorInvalidDevice; }
bool skinny_m_fits(const GemmArgs&) { return false; }
hipError_t launch_skinny_m(const GemmArgs&, hipStream_t) { return hipErrorInvalidDevice; }
bool skinny_n_fits(const GemmArgs&) { return false; }
hipError_t launch_skinny_n(const GemmArgs&, hipStream_t) { return hipErrorInvalidDevice; }
hipError_t launch_micro4x4(int, const float*, const float*, float*, hipStream_t) {
    return hipErrorInvalidDevice;
}
hipError_t launch_lowp(const LowpArgs&, Lowp, hipStream_t) { return hipErrorInvalidDevice; }
int valu_tile_count() { return 15; }
const char* valu_tile_name(int tile) { return tile >= 0 && tile < 15 ? "stub" : nullptr; }
hipError_t launch_valu_tile(const GemmArgs&, int, hipStream_t) { return hipErrorInvalidDevice; }
}  // namespace sgemm

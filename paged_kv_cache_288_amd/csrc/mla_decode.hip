// Latent (MLA) decode attention: placeholder launcher until the MFMA kernel lands.
#include "pkv_device.hpp"
#include "pkv_launch.hpp"

namespace pkv {

hipError_t launch_mla_decode(const MlaArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv

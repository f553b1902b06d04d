#include "device_common.hpp"
#include "launch.hpp"
namespace libscan {
size_t radix_body_bytes(uint64_t, int) { return 0; }
hipError_t launch_radix(const uint32_t *, int32_t *, uint64_t, int, const Scratch &, hipStream_t) { return hipErrorNotSupported; }
}

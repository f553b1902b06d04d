#include "device_common.hpp"
#include "launch.hpp"
namespace libscan {
size_t segscan_body_bytes(uint64_t, uint64_t) { return 0; }
hipError_t launch_segscan(const uint32_t *, uint32_t *, uint64_t, uint64_t, uint32_t *, const Scratch &, hipStream_t) { return hipErrorNotSupported; }
}

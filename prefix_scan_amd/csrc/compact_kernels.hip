#include "device_common.hpp"
#include "launch.hpp"
namespace libscan {
size_t compact_body_bytes(uint64_t) { return 0; }
hipError_t launch_compact(const int32_t *, int32_t *, uint64_t, const Scratch &, uint32_t *, hipStream_t) { return hipErrorNotSupported; }
}

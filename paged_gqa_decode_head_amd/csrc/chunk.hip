// Causal chunk attention over the paged cache (placeholder translation unit).
#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
hipError_t launch_chunk(const PoolGeom&, const ChunkArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pgqa

// Host-side helpers shared by the library's translation units.
#pragma once

namespace mxq {

// Compute-unit count of the current device, queried once per device.
int device_cu_count();

}  // namespace mxq

// Host-side helpers shared by the library's translation units.
#pragma once

#include <stdint.h>

#include "mxq.h"

namespace mxq {

// Compute-unit count of the current device, queried once per device.
int device_cu_count();

// The fused smooth + rotate + MXFP4 path behind mxq_rotate_quant and its
// variants (tiled: fragment-tiled output).
mxq_status rotate_impl(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels, int64_t stride,
                       const float* lambda, const uint16_t* r_hat, uint8_t* codes, uint8_t* scales, float* y,
                       void* stream, bool tiled);

}  // namespace mxq

// Host-side offline calibration (internal).
#pragma once
#include <stdint.h>

namespace oscar {
// Rotations (the public OSCAR_ROT_* values).
enum CalibRotation { kRotSpectral = 0, kRotKeyAttn = 1, kRotHadamard = 2, kRotIdentity = 3 };

// Returns 0 on success, -1 when an input or a resulting clip threshold is not
// finite, not positive, or above 65504.
int calibrate_layer(int hq, int hkv, int hadamard_block, float percentile, int rotation, const float* q,
                    const float* k, const float* v, int64_t n, float* rot_k, float* rot_v, float* clip_k,
                    float* clip_v);
}  // namespace oscar

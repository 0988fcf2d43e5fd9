// Host-side offline calibration (internal).
#pragma once
#include <stdint.h>

namespace oscar {
// Rotations (the public OSCAR_ROT_* values).
enum CalibRotation { kRotSpectral = 0, kRotKeyAttn = 1, kRotHadamard = 2, kRotIdentity = 3 };

// One calibration for n_layers layers of n tokens each (q [L][n][hq][128],
// k, v [L][n][hkv][128]); per_kv_head: one output set per KV head
// (rot [hkv][128][128], clip [hkv][128]), otherwise one set.  Returns 0 on
// success, -1 when an input or a resulting clip threshold is not finite, not
// positive, or above 65504, -2 for an unknown rotation.
int calibrate_layers(int hq, int hkv, int n_layers, int hadamard_block, float percentile, int rotation,
                     bool per_kv_head, const float* q, const float* k, const float* v, int64_t n, float* rot_k,
                     float* rot_v, float* clip_k, float* clip_v);
}  // namespace oscar

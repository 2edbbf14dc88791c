// Device helpers shared by every kernel that applies the 3D rotary embedding
// (in place, and fused into the cache write), so that both produce the same
// bits: the token position, the angle and the rotation of one pair are
// written once here, with floating-point contraction off, so that no caller's
// context can fuse a multiply into a neighbouring add differently. The
// convention is the one documented in include/wf.h (the pages do not
// describe positional encoding).
#pragma once

#include "wf_internal.h"

namespace wf {

// Position (frame, row, column) of token u of global chunk g; tokens inside a
// chunk are ordered frame, then row, then column.
__device__ __forceinline__ void rope_token_pos(int g, int u, int fpc, int gh, int gw, float pos[3]) {
  const int plane = gh * gw;
  pos[0] = (float)(fpc * g + u / plane);
  pos[1] = (float)((u / gw) % gh);
  pos[2] = (float)(u % gw);
}

// sin and cos of the angle of pair pr at that position (fp32 product pos * inv_freq).
__device__ __forceinline__ void rope_sincos(const float pos[3], const RopeTable& tab, int pr, float& sn, float& cs) {
#pragma clang fp contract(off)
  const float phi = pos[tab.axis[pr]] * tab.inv_freq[pr];
  sincosf(phi, &sn, &cs);
}

// Rotates the interleaved pair (a, b) by the angle with this sin and cos (fp32
// arithmetic, result rounded to T).
template <typename T>
__device__ __forceinline__ void rope_rotate_pair(T& a, T& b, float cs, float sn) {
#pragma clang fp contract(off)
  const float x0 = (float)a, x1 = (float)b;
  a = (T)(x0 * cs - x1 * sn);
  b = (T)(x0 * sn + x1 * cs);
}

}  // namespace wf

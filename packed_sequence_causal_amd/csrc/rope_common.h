// Rotary position embedding arithmetic shared by the rotation kernel
// (rope.hip) and the attention kernels that rotate inside their loads and
// epilogues, so a rotation gives the same bits wherever it runs.
//
// Rotate-half form (XTuner sequence-parallel page, section "实现方案",
// apply_rotary_pos_emb(q, k, cos, sin)): dims i and i + D/2 of a head turn by
// theta_i = pos * base^(-2i/D), pos = the token's offset inside its segment
// (the packer's indexes: InternEvo "数据加载与流程", section
// "获取Dataloader数据").  The angle is formed and reduced modulo 2*pi in fp64
// (an fp32 product pos * freq would be off by ~0.01 rad near position 10^5),
// then sin and cos are taken in fp32 on an argument in [-pi, pi]; the turn
// itself is two fp32 fmas.  The inverse turn (the backward) is the turn by
// -theta.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace psc {

constexpr double kTwoPiHi = 6.283185307179586;       // nearest double to 2*pi
constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;

// cos and sin of pos * inv_freq (sin negated for the inverse turn).
__device__ __forceinline__ void rope_cs(int32_t pos, double inv_freq, bool inverse, float& c, float& s) {
  const double th = (double)pos * inv_freq;
  const double k = rint(th * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, th);
  r = fma(-k, kTwoPiLo, r);
  float sv, cv;
  sincosf((float)r, &sv, &cv);
  c = cv;
  s = inverse ? -sv : sv;
}

// (a1, a2) = dims (i, i + D/2) turned by the angle whose cos, sin are (c, s).
__device__ __forceinline__ void rope_turn(float a1, float a2, float c, float s, float& y1, float& y2) {
  y1 = __builtin_fmaf(a1, c, -a2 * s);
  y2 = __builtin_fmaf(a2, c, a1 * s);
}

}  // namespace psc

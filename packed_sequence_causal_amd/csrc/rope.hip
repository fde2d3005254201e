// Rotary position embedding of packed rows, in place on q and k, with each
// token's position taken from the packer's `indexes` (its offset inside its
// segment: InternEvo "数据加载与流程", section "获取Dataloader数据").  The
// rotation is the rotate-half form that an apply_rotary_pos_emb(q, k, cos,
// sin) call applies (XTuner sequence-parallel page, section "实现方案"): dims
// i and i + D/2 turn by theta_i = pos * base^(-2i/D).
//
// HBM-bound: every element is read and written once.  One thread owns one
// token and PP consecutive pairs (16-byte loads of each half), computes their
// angles once and applies them to every head of q and then of k.  The angle
// is formed and reduced modulo 2*pi in fp64 (an fp32 product pos * freq would
// be off by ~0.01 rad near position 10^5), then sin and cos are taken in fp32
// on an argument in [-pi, pi].
#include "attn_common.h"
#include "psc_internal.h"

#include <type_traits>

namespace psc {
namespace {

constexpr int kRopeThreads = 256;
constexpr double kTwoPiHi = 6.283185307179586;        // nearest double to 2*pi
constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;

template <typename E>
struct Vec16;
template <>
struct Vec16<bf16> {
  typedef bf16x8 type;
};
template <>
struct Vec16<float> {
  typedef f32x4 type;
};

template <typename E, int D>
__global__ void __launch_bounds__(kRopeThreads) k_rope(RopeArgs a) {
  constexpr int PP = 16 / sizeof(E);  // pairs per thread
  constexpr int TPT = (D / 2) / PP;   // threads per token
  typedef typename Vec16<E>::type V;
  const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int64_t t = gid / TPT;
  if (t >= a.T) return;
  const int i0 = (int)(gid - t * TPT) * PP;
  const double pos = (double)a.pos[t];
  float c[PP], s[PP];
#pragma unroll
  for (int j = 0; j < PP; ++j) {
    const double th = pos * a.inv_freq[i0 + j];
    const double k = rint(th * kInvTwoPi);
    double r = fma(-k, kTwoPiHi, th);
    r = fma(-k, kTwoPiLo, r);
    sincosf((float)r, &s[j], &c[j]);
    if (a.inverse) s[j] = -s[j];
  }
  // NH heads per step: all their loads are issued before the first use
  auto rotate_heads = [&](E* row, auto nh_c) {
    constexpr int NH = decltype(nh_c)::value;
    V x1[NH], x2[NH];
#pragma unroll
    for (int u = 0; u < NH; ++u) {
      x1[u] = *reinterpret_cast<const V*>(row + u * D);
      x2[u] = *reinterpret_cast<const V*>(row + u * D + D / 2);
    }
#pragma unroll
    for (int u = 0; u < NH; ++u) {
      V y1, y2;
#pragma unroll
      for (int j = 0; j < PP; ++j) {
        const float a1 = (float)x1[u][j], a2 = (float)x2[u][j];
        y1[j] = (E)__builtin_fmaf(a1, c[j], -a2 * s[j]);
        y2[j] = (E)__builtin_fmaf(a2, c[j], a1 * s[j]);
      }
      *reinterpret_cast<V*>(row + u * D) = y1;
      *reinterpret_cast<V*>(row + u * D + D / 2) = y2;
    }
  };
  auto rotate = [&](void* base, int64_t stride, int32_t heads) {
    E* row = static_cast<E*>(base) + t * stride + i0;
    int32_t h = 0;
    for (; h + 4 <= heads; h += 4, row += 4 * D) rotate_heads(row, std::integral_constant<int, 4>{});
    for (; h < heads; ++h, row += D) rotate_heads(row, std::integral_constant<int, 1>{});
  };
  rotate(a.q, a.sq, a.hq);
  if (a.k) rotate(a.k, a.sk, a.hkv);
}

template <typename E, int D>
hipError_t launch_typed(const RopeArgs& a, hipStream_t stream) {
  constexpr int TPT = (D / 2) / (16 / sizeof(E));
  const int64_t threads = a.T * TPT;
  const uint64_t blocks = (uint64_t)((threads + kRopeThreads - 1) / kRopeThreads);
  k_rope<E, D><<<(unsigned)blocks, kRopeThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  ScopedKernelTimer timed(kTimeRope, stream);
  if (a.dtype == 1) {
    if (a.d == 128) return launch_typed<bf16, 128>(a, stream);
    if (a.d == 64) return launch_typed<bf16, 64>(a, stream);
    return launch_typed<bf16, 32>(a, stream);
  }
  if (a.d == 128) return launch_typed<float, 128>(a, stream);
  if (a.d == 64) return launch_typed<float, 64>(a, stream);
  return launch_typed<float, 32>(a, stream);
}

}  // namespace psc

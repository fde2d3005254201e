// Rotary position embedding of packed rows, in place on q and k, with each
// token's position taken from the packer's `indexes` (its offset inside its
// segment: InternEvo "数据加载与流程", section "获取Dataloader数据").  The
// rotation is the rotate-half form that an apply_rotary_pos_emb(q, k, cos,
// sin) call applies (XTuner sequence-parallel page, section "实现方案"): dims
// i and i + D/2 turn by theta_i = pos * base^(-2i/D).
//
// HBM-bound: every element is read and written once; each token's angles are
// formed once per workgroup and shared through LDS (see k_rope).  The angle
// is formed and reduced modulo 2*pi in fp64 (an fp32 product pos * freq would
// be off by ~0.01 rad near position 10^5), then sin and cos are taken in fp32
// on an argument in [-pi, pi].
#include "attn_common.h"
#include "psc_internal.h"
#include "rope_common.h"

#include <algorithm>
#include <type_traits>

namespace psc {
namespace {

constexpr int kRopeThreads = 256;

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

// One workgroup rotates kTokPerWg consecutive tokens (one: measured fastest,
// against 2, 4 and 8).  First its threads form the tokens' D/2 angles (fp64
// product and reduction, fp32 sin/cos) into LDS; then the workgroup walks the
// tokens' pair chunks -- PP
// consecutive pairs of one head: a 16-byte load from each half -- thread t
// taking chunks t, t + kRopeThreads, ..., with every load in flight before
// the first rotation.  Consecutive threads take consecutive chunks of one
// head row, so a wave covers whole 2*D-byte rows of consecutive heads.
constexpr int kTokPerWg = 1;

template <typename E, int D>
__global__ void __launch_bounds__(kRopeThreads) k_rope(RopeArgs a) {
  constexpr int PP = 16 / sizeof(E);       // pairs per chunk
  constexpr int CPH = (D / 2) / PP;        // chunks per head
  typedef typename Vec16<E>::type V;
  __shared__ float cs_s[kTokPerWg][D / 2], sn_s[kTokPerWg][D / 2];
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerWg;
  const int ntok = (int)min<int64_t>(kTokPerWg, a.T - t0);
  for (int x = threadIdx.x; x < kTokPerWg * (D / 2); x += kRopeThreads) {
    const int tk = x / (D / 2), i = x % (D / 2);
    float c = 1.f, sv = 0.f;
    if (tk < ntok) rope_cs(a.pos[t0 + tk], a.inv_freq[i], a.inverse != 0, c, sv);
    cs_s[tk][i] = c;
    sn_s[tk][i] = sv;
  }
  __syncthreads();
  // chunk index: token-major, then q heads then k heads, then chunk in head
  const int cq = a.hq * CPH, ck = a.hkv * CPH, cpt = cq + ck;
  const int total = ntok * cpt;
  constexpr int NB = 4;  // chunks per thread in flight
  for (int base = threadIdx.x; base < total; base += NB * kRopeThreads) {
    E* ptr[NB];
    int ii[NB], tkk[NB];
    V x1[NB], x2[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int c = base + u * kRopeThreads;
      ptr[u] = nullptr;
      if (c < total) {
        const int tk = c / cpt, r = c - tk * cpt;
        const bool isq = r < cq;
        const int rr = isq ? r : r - cq;
        const int hh = rr / CPH, j = rr - hh * CPH;
        ptr[u] = static_cast<E*>(isq ? a.q : a.k) + (t0 + tk) * (isq ? a.sq : a.sk) + (int64_t)hh * D + j * PP;
        ii[u] = j * PP;
        tkk[u] = tk;
        x1[u] = *reinterpret_cast<const V*>(ptr[u]);
        x2[u] = *reinterpret_cast<const V*>(ptr[u] + D / 2);
      }
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (!ptr[u]) continue;
      V y1, y2;
#pragma unroll
      for (int e = 0; e < PP; ++e) {
        const float c = cs_s[tkk[u]][ii[u] + e], sv = sn_s[tkk[u]][ii[u] + e];
        float r1, r2;
        rope_turn((float)x1[u][e], (float)x2[u][e], c, sv, r1, r2);
        y1[e] = (E)r1;
        y2[e] = (E)r2;
      }
      *reinterpret_cast<V*>(ptr[u]) = y1;
      *reinterpret_cast<V*>(ptr[u] + D / 2) = y2;
    }
  }
}

template <typename E, int D>
hipError_t launch_typed(const RopeArgs& a, hipStream_t stream) {
  const uint64_t blocks = (uint64_t)((a.T + kTokPerWg - 1) / kTokPerWg);
  k_rope<E, D><<<(unsigned)blocks, kRopeThreads, 0, stream>>>(a);
  return hipGetLastError();
}

// cos and sin of every (position, frequency) pair for positions [0, n_pos):
// table[pos * (D/2) + i] = (cos, sin) of pos * inv_freq[i], the turn the
// attention kernels apply inside their loads and epilogues.
__global__ void __launch_bounds__(kRopeThreads) k_rope_table(RopeArgs a, int32_t n_pos, float2* table) {
  const int half = a.d / 2;
  const int64_t n = (int64_t)n_pos * half;
  for (int64_t x = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x; x < n; x += (int64_t)gridDim.x * kRopeThreads) {
    const int32_t pos = (int32_t)(x / half);
    const int i = (int)(x - (int64_t)pos * half);
    float c, sv;
    rope_cs(pos, a.inv_freq[i], false, c, sv);
    table[x] = make_float2(c, sv);
  }
}

}  // namespace

hipError_t launch_rope_table(const RopeArgs& a, int32_t n_pos, float2* table, hipStream_t stream) {
  const int64_t n = (int64_t)n_pos * (a.d / 2);
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + kRopeThreads - 1) / kRopeThreads, 4096);
  k_rope_table<<<blocks, kRopeThreads, 0, stream>>>(a, n_pos, table);
  return hipGetLastError();
}

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

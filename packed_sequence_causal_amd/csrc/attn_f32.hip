// Document-causal attention in true fp32 (no bf16 or tf32 rounding anywhere).
//
// Path for fp32 inputs.  Each (query row, head) of the forward and dQ, and
// each (key row, key/value head) of dK/dV, belongs to a group of 16 lanes of
// one wave: lane r of the group holds elements r E .. r E + E - 1 (E = D/16)
// of the row's vectors, a dot product is a per-lane partial sum reduced over
// the group, and a thread holds only E elements of any vector.  Scores,
// softmax and products are fp32 FMA; exp and log are the full-precision
// library functions.  Each group visits only
// its own document's causal range ("Sample Packing：长序列 LLM 训练的 Attention
// 问题及优化", section 三: one causal triangle per document), so the cost is
// the in-document work, without tiles.
#include <cmath>

#include "psc_internal.h"

namespace psc {
namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 16;                  // lanes per row
constexpr int kRows = kThreads / kGroup;   // rows per workgroup

// Segment holding token t: last s with cu[s] <= t.
__device__ inline int32_t seg_of(const int32_t* cu, int32_t n_seg, int64_t t) {
  int32_t lo = 0, hi = n_seg;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Sum over the 16 lanes of a group (xor butterfly inside 16-lane rows).
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = kGroup / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, kGroup);
  return x;
}

struct F32Params {
  const float *q, *k, *v, *o, *dout, *lse_in;
  float *out, *lse, *Dbuf, *dq, *dk, *dv;
  int64_t sq, sk, sv, so, sdo, T;
  const int32_t* cu;
  int32_t n_seg, hq, hkv, group;
  float scale;
};

// E = D / 16 consecutive elements of a row, from lane r's slice.
template <int E>
__device__ __forceinline__ void load_slice(const float* row, int r, float (&x)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = row[r * E + e];
}

template <int D>
__global__ void __launch_bounds__(kThreads) k_f32_fwd(F32Params p) {
  constexpr int E = D / kGroup;
  const int r = threadIdx.x % kGroup;
  const int64_t t = (int64_t)blockIdx.x * kRows + threadIdx.x / kGroup;
  const int32_t head = blockIdx.y;
  if (t >= p.T) return;  // whole groups leave together
  const int32_t s = seg_of(p.cu, p.n_seg, t);
  const int64_t s0 = min(max((int64_t)p.cu[s], (int64_t)0), t);
  const int32_t g = head / p.group;
  float qv[E], acc[E];
  load_slice<E>(p.q + t * p.sq + (int64_t)head * D, r, qv);
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int64_t j = s0; j <= t; ++j) {
    float kv[E], vv[E];
    load_slice<E>(p.k + j * p.sk + (int64_t)g * D, r, kv);
    load_slice<E>(p.v + j * p.sv + (int64_t)g * D, r, vv);
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) x = fmaf(qv[e], kv[e], x);
    x = group_sum(x) * p.scale;
    const float mn = fmaxf(m, x);
    const float a = expf(m - mn);
    const float ex = expf(x - mn);
    l = l * a + ex;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(ex, vv[e], acc[e] * a);
    m = mn;
  }
  float* orow = p.out + t * p.so + (int64_t)head * D;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[r * E + e] = acc[e] / l;
  if (r == 0) p.lse[(int64_t)head * p.T + t] = m + logf(l);
}

template <int D>
__global__ void __launch_bounds__(kThreads) k_f32_pre(F32Params p) {
  constexpr int E = D / kGroup;
  const int r = threadIdx.x % kGroup;
  const int64_t t = (int64_t)blockIdx.x * kRows + threadIdx.x / kGroup;
  const int32_t head = blockIdx.y;
  if (t >= p.T) return;
  float ov[E], dv[E];
  load_slice<E>(p.o + t * p.so + (int64_t)head * D, r, ov);
  load_slice<E>(p.dout + t * p.sdo + (int64_t)head * D, r, dv);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc = fmaf(ov[e], dv[e], acc);
  acc = group_sum(acc);
  if (r == 0) p.Dbuf[(int64_t)head * p.T + t] = acc;
}

template <int D>
__global__ void __launch_bounds__(kThreads) k_f32_dq(F32Params p) {
  constexpr int E = D / kGroup;
  const int r = threadIdx.x % kGroup;
  const int64_t t = (int64_t)blockIdx.x * kRows + threadIdx.x / kGroup;
  const int32_t head = blockIdx.y;
  if (t >= p.T) return;
  const int32_t s = seg_of(p.cu, p.n_seg, t);
  const int64_t s0 = min(max((int64_t)p.cu[s], (int64_t)0), t);
  const int32_t g = head / p.group;
  float qv[E], dov[E], acc[E];
  load_slice<E>(p.q + t * p.sq + (int64_t)head * D, r, qv);
  load_slice<E>(p.dout + t * p.sdo + (int64_t)head * D, r, dov);
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const float lse = p.lse_in[(int64_t)head * p.T + t];
  const float Dt = p.Dbuf[(int64_t)head * p.T + t];
  for (int64_t j = s0; j <= t; ++j) {
    float kv[E], vv[E];
    load_slice<E>(p.k + j * p.sk + (int64_t)g * D, r, kv);
    load_slice<E>(p.v + j * p.sv + (int64_t)g * D, r, vv);
    float x = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      x = fmaf(qv[e], kv[e], x);
      dp = fmaf(dov[e], vv[e], dp);
    }
    x = group_sum(x);
    dp = group_sum(dp);
    const float pr = expf(x * p.scale - lse);
    const float ds = pr * (dp - Dt);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, kv[e], acc[e]);
  }
  float* out = p.dq + (t * p.hq + head) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) out[r * E + e] = acc[e] * p.scale;
}

template <int D>
__global__ void __launch_bounds__(kThreads) k_f32_dkdv(F32Params p) {
  constexpr int E = D / kGroup;
  const int r = threadIdx.x % kGroup;
  const int64_t j = (int64_t)blockIdx.x * kRows + threadIdx.x / kGroup;
  const int32_t g = blockIdx.y;
  if (j >= p.T) return;
  const int32_t s = seg_of(p.cu, p.n_seg, j);
  const int64_t e_end = min(max((int64_t)p.cu[s + 1], j + 1), p.T);
  float kv[E], vv[E], dk[E], dv[E];
  load_slice<E>(p.k + j * p.sk + (int64_t)g * D, r, kv);
  load_slice<E>(p.v + j * p.sv + (int64_t)g * D, r, vv);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  for (int32_t hh = 0; hh < p.group; ++hh) {
    const int32_t head = g * p.group + hh;
    for (int64_t i = j; i < e_end; ++i) {
      float qv[E], dov[E];
      load_slice<E>(p.q + i * p.sq + (int64_t)head * D, r, qv);
      load_slice<E>(p.dout + i * p.sdo + (int64_t)head * D, r, dov);
      float x = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        x = fmaf(qv[e], kv[e], x);
        dp = fmaf(dov[e], vv[e], dp);
      }
      x = group_sum(x);
      dp = group_sum(dp);
      const float pr = expf(x * p.scale - p.lse_in[(int64_t)head * p.T + i]);
      const float ds = pr * (dp - p.Dbuf[(int64_t)head * p.T + i]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dv[e] = fmaf(pr, dov[e], dv[e]);
        dk[e] = fmaf(ds, qv[e], dk[e]);
      }
    }
  }
  float* dko = p.dk + (j * p.hkv + g) * D;
  float* dvo = p.dv + (j * p.hkv + g) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dko[r * E + e] = dk[e] * p.scale;
    dvo[r * E + e] = dv[e];
  }
}

template <int D>
hipError_t fwd_d(const F32Params& p, hipStream_t st) {
  dim3 grid((unsigned)((p.T + kRows - 1) / kRows), (unsigned)p.hq);
  k_f32_fwd<D><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const F32Params& p, hipStream_t st) {
  dim3 gq((unsigned)((p.T + kRows - 1) / kRows), (unsigned)p.hq);
  dim3 gk((unsigned)((p.T + kRows - 1) / kRows), (unsigned)p.hkv);
  k_f32_pre<D><<<gq, kThreads, 0, st>>>(p);
  k_f32_dq<D><<<gq, kThreads, 0, st>>>(p);
  k_f32_dkdv<D><<<gk, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnFwdArgs& a, hipStream_t stream) {
  const AttnDims& d = a.dims;
  if (d.T == 0) return hipSuccess;
  F32Params p{};
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.out = static_cast<float*>(a.out);
  p.lse = a.lse;
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  p.T = d.T;
  p.cu = a.cu;
  p.n_seg = d.n_seg;
  p.hq = d.hq;
  p.hkv = d.hkv;
  p.group = d.hq / d.hkv;
  p.scale = d.scale;
  switch (d.d) {
    case 32: return fwd_d<32>(p, stream);
    case 64: return fwd_d<64>(p, stream);
    default: return fwd_d<128>(p, stream);
  }
}

hipError_t launch_attn_bwd_f32(const AttnBwdArgs& a, hipStream_t stream) {
  const AttnDims& d = a.dims;
  if (d.T == 0) return hipSuccess;
  F32Params p{};
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<const float*>(a.o);
  p.dout = static_cast<const float*>(a.dout);
  p.lse_in = a.lse;
  p.Dbuf = static_cast<float*>(a.workspace);
  p.dq = static_cast<float*>(a.dq);
  p.dk = static_cast<float*>(a.dk);
  p.dv = static_cast<float*>(a.dv);
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  p.sdo = a.sdo;
  p.T = d.T;
  p.cu = a.cu;
  p.n_seg = d.n_seg;
  p.hq = d.hq;
  p.hkv = d.hkv;
  p.group = d.hq / d.hkv;
  p.scale = d.scale;
  switch (d.d) {
    case 32: return bwd_d<32>(p, stream);
    case 64: return bwd_d<64>(p, stream);
    default: return bwd_d<128>(p, stream);
  }
}

}  // namespace psc

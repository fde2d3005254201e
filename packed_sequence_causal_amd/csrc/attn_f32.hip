// Document-causal attention in true fp32 (no bf16 or tf32 rounding anywhere).
//
// Small-problem path for fp32 inputs: one thread per (query row, head) for the
// forward and dQ, one thread per (key row, key/value head) for dK/dV.  Scores,
// softmax and products are fp32 FMA; exp and log are the full-precision
// library functions.  Each thread visits only its own document's causal range
// ("Sample Packing：长序列 LLM 训练的 Attention 问题及优化", section 三: one causal
// triangle per document), so the cost is the in-document work, without tiles.
#include <cmath>

#include "psc_internal.h"

namespace psc {
namespace {

constexpr int kThreads = 128;

// Segment holding token t: last s with cu[s] <= t.
__device__ inline int32_t seg_of(const int32_t* cu, int32_t n_seg, int64_t t) {
  int32_t lo = 0, hi = n_seg;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

struct F32Params {
  const float *q, *k, *v, *o, *dout, *lse_in;
  float *out, *lse, *Dbuf, *dq, *dk, *dv;
  int64_t sq, sk, sv, so, sdo, T;
  const int32_t* cu;
  int32_t n_seg, hq, hkv, group;
  float scale;
};

template <int D>
__global__ void __launch_bounds__(kThreads) k_f32_fwd(F32Params p) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int32_t head = blockIdx.y;
  if (t >= p.T) return;
  const int32_t s = seg_of(p.cu, p.n_seg, t);
  const int64_t s0 = min(max((int64_t)p.cu[s], (int64_t)0), t);
  const int32_t g = head / p.group;
  float qv[D], acc[D];
  const float* qr = p.q + t * p.sq + (int64_t)head * D;
  for (int d = 0; d < D; ++d) {
    qv[d] = qr[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int64_t j = s0; j <= t; ++j) {
    const float* kr = p.k + j * p.sk + (int64_t)g * D;
    float x = 0.f;
    for (int d = 0; d < D; ++d) x = fmaf(qv[d], kr[d], x);
    x *= p.scale;
    const float mn = fmaxf(m, x);
    const float a = expf(m - mn);
    const float e = expf(x - mn);
    l = l * a + e;
    const float* vr = p.v + j * p.sv + (int64_t)g * D;
    for (int d = 0; d < D; ++d) acc[d] = fmaf(e, vr[d], acc[d] * a);
    m = mn;
  }
  float* orow = p.out + t * p.so + (int64_t)head * D;
  for (int d = 0; d < D; ++d) orow[d] = acc[d] / l;
  p.lse[(int64_t)head * p.T + t] = m + logf(l);
}

template <int D>
__global__ void __launch_bounds__(kThreads) k_f32_pre(F32Params p) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int32_t head = blockIdx.y;
  if (t >= p.T) return;
  const float* orow = p.o + t * p.so + (int64_t)head * D;
  const float* drow = p.dout + t * p.sdo + (int64_t)head * D;
  float acc = 0.f;
  for (int d = 0; d < D; ++d) acc = fmaf(orow[d], drow[d], acc);
  p.Dbuf[(int64_t)head * p.T + t] = acc;
}

template <int D>
__global__ void __launch_bounds__(kThreads) k_f32_dq(F32Params p) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int32_t head = blockIdx.y;
  if (t >= p.T) return;
  const int32_t s = seg_of(p.cu, p.n_seg, t);
  const int64_t s0 = min(max((int64_t)p.cu[s], (int64_t)0), t);
  const int32_t g = head / p.group;
  float qv[D], dov[D], acc[D];
  const float* qr = p.q + t * p.sq + (int64_t)head * D;
  const float* dr = p.dout + t * p.sdo + (int64_t)head * D;
  for (int d = 0; d < D; ++d) {
    qv[d] = qr[d];
    dov[d] = dr[d];
    acc[d] = 0.f;
  }
  const float lse = p.lse_in[(int64_t)head * p.T + t];
  const float Dt = p.Dbuf[(int64_t)head * p.T + t];
  for (int64_t j = s0; j <= t; ++j) {
    const float* kr = p.k + j * p.sk + (int64_t)g * D;
    const float* vr = p.v + j * p.sv + (int64_t)g * D;
    float x = 0.f, dp = 0.f;
    for (int d = 0; d < D; ++d) {
      x = fmaf(qv[d], kr[d], x);
      dp = fmaf(dov[d], vr[d], dp);
    }
    const float pr = expf(x * p.scale - lse);
    const float ds = pr * (dp - Dt);
    for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, kr[d], acc[d]);
  }
  float* out = p.dq + (t * p.hq + head) * D;
  for (int d = 0; d < D; ++d) out[d] = acc[d] * p.scale;
}

template <int D>
__global__ void __launch_bounds__(kThreads) k_f32_dkdv(F32Params p) {
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int32_t g = blockIdx.y;
  if (j >= p.T) return;
  const int32_t s = seg_of(p.cu, p.n_seg, j);
  const int64_t e = min(max((int64_t)p.cu[s + 1], j + 1), p.T);
  float kv[D], vv[D], dk[D], dv[D];
  const float* kr = p.k + j * p.sk + (int64_t)g * D;
  const float* vr = p.v + j * p.sv + (int64_t)g * D;
  for (int d = 0; d < D; ++d) {
    kv[d] = kr[d];
    vv[d] = vr[d];
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  for (int32_t hh = 0; hh < p.group; ++hh) {
    const int32_t head = g * p.group + hh;
    for (int64_t i = j; i < e; ++i) {
      const float* qr = p.q + i * p.sq + (int64_t)head * D;
      const float* dr = p.dout + i * p.sdo + (int64_t)head * D;
      float x = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        x = fmaf(qr[d], kv[d], x);
        dp = fmaf(dr[d], vv[d], dp);
      }
      const float pr = expf(x * p.scale - p.lse_in[(int64_t)head * p.T + i]);
      const float ds = pr * (dp - p.Dbuf[(int64_t)head * p.T + i]);
      for (int d = 0; d < D; ++d) {
        dv[d] = fmaf(pr, dr[d], dv[d]);
        dk[d] = fmaf(ds, qr[d], dk[d]);
      }
    }
  }
  float* dko = p.dk + (j * p.hkv + g) * D;
  float* dvo = p.dv + (j * p.hkv + g) * D;
  for (int d = 0; d < D; ++d) {
    dko[d] = dk[d] * p.scale;
    dvo[d] = dv[d];
  }
}

template <int D>
hipError_t fwd_d(const F32Params& p, hipStream_t st) {
  dim3 grid((unsigned)((p.T + kThreads - 1) / kThreads), (unsigned)p.hq);
  k_f32_fwd<D><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const F32Params& p, hipStream_t st) {
  dim3 gq((unsigned)((p.T + kThreads - 1) / kThreads), (unsigned)p.hq);
  dim3 gk((unsigned)((p.T + kThreads - 1) / kThreads), (unsigned)p.hkv);
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

// Document-causal attention backward, bf16 operands / fp32 accumulate, gfx950.
//
// Gradients of sum(dO * O) for O = softmax(scale * Q K^T restricted to each
// document's causal triangle) V, with P recomputed from the forward's lse:
//   D_i   = <dO_i, O_i>                      (k_bwd_pre)
//   P     = exp(scale * q_i.k_j - lse_i)      (recomputed)
//   dP    = dO V^T,   dS = P * (dP - D)
//   dV    = P^T dO,   dK = scale dS^T Q       (k_bwd_dkdv: one workgroup per
//                                              128-key tile and key/value head;
//                                              loops over the head group's
//                                              query heads and the query blocks
//                                              from the tile to the document end)
//   dQ    = scale dS K                        (k_bwd_dq: one workgroup per
//                                              128-row query tile and query head;
//                                              loops over key blocks up to the
//                                              diagonal)
// Splitting dQ from dK/dV recomputes S and dP once more but needs no atomics:
// every output element is written once, and results are deterministic.
// Both loops visit only tiles inside a document's causal triangle ("Sample
// Packing：长序列 LLM 训练的 Attention 问题及优化", section 5.1).
#include "attn_common.h"
#include "psc_internal.h"

namespace psc {
namespace {

constexpr int kThreads = 256;
constexpr int kBQ = 128;   // dQ kernel: query rows per workgroup (4 waves x 32)
constexpr int kBNq = 64;   // dQ kernel: keys per block
constexpr int kBKV = 128;  // dK/dV kernel: keys per workgroup (4 waves x 32)
constexpr int kBMk = 64;   // dK/dV kernel: queries per block

struct BwdParams {
  const bf16 *q, *k, *v, *o, *dout;
  const float* lse;
  float* Dbuf;  // [hq][T]
  float *dq, *dk, *dv;
  int64_t sq, sk, sv, so, sdo, T;
  const int32_t* cu;
  const int32_t* items;
  const int32_t* n_items;
  int32_t hq, hkv, group;
  float scale, scale_log2;
};

// D[h][t] = sum_d dO[t,h,d] * O[t,h,d] in fp32; 16 lanes per (token, head)
// for D = 128 (8 per lane), 8 lanes for D = 64.
template <int D>
__global__ void __launch_bounds__(kThreads) k_bwd_pre(BwdParams p) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = gid / LPR;  // row = t * hq + h
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (row < p.T * p.hq) {
    const int64_t t = row / p.hq;
    const int h = (int)(row % p.hq);
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p.o + t * p.so + (int64_t)h * D + part * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(p.dout + t * p.sdo + (int64_t)h * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (row < p.T * p.hq && part == 0) {
    const int64_t t = row / p.hq;
    const int h = (int)(row % p.hq);
    p.Dbuf[(int64_t)h * p.T + t] = acc;
  }
}

template <int D>
struct KSt {
  static constexpr int S = D + 8;
};

// ---------------------------------------------------------------------- dQ
template <int D>
__global__ void __launch_bounds__(kThreads, 2) k_bwd_dq(BwdParams p) {
  constexpr int S = KSt<D>::S;
  __shared__ __attribute__((aligned(16))) bf16 Ks[kBNq * S];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kBNq * S];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;
  const uint32_t b = xcd_group_remap(blockIdx.x, gridDim.x, (uint32_t)p.group);
  const uint32_t item = b / (uint32_t)p.hq, head = b % (uint32_t)p.hq;
  if ((int32_t)item >= *p.n_items) return;
  const int32_t seg = p.items[2 * item], tile = p.items[2 * item + 1];
  const int32_t s0 = min(max(p.cu[seg], 0), (int32_t)p.T);
  const int32_t L = min(max(p.cu[seg + 1], s0), (int32_t)p.T) - s0;
  const int32_t q0 = tile * kBQ;
  if (q0 >= L) return;
  const int32_t kvh = (int32_t)head / p.group;

  const bf16* Kp = p.k + (int64_t)s0 * p.sk + (int64_t)kvh * D;
  const bf16* Vp = p.v + (int64_t)s0 * p.sv + (int64_t)kvh * D;

  const int32_t qrow = q0 + 32 * w + lq;
  const bool qvalid = qrow < L;
  bf16x8 qf[D / 16], df[D / 16];
  {
    const bf16* Qr = p.q + (int64_t)(s0 + qrow) * p.sq + (int64_t)head * D;
    const bf16* Dr = p.dout + (int64_t)(s0 + qrow) * p.sdo + (int64_t)head * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = qvalid ? *reinterpret_cast<const bf16x8*>(Qr + 16 * kk + 8 * h) : bf16x8{};
      df[kk] = qvalid ? *reinterpret_cast<const bf16x8*>(Dr + 16 * kk + 8 * h) : bf16x8{};
    }
  }
  const float lse2 = qvalid ? p.lse[(int64_t)head * p.T + s0 + qrow] * kLog2e : 0.f;
  const float Drow = qvalid ? p.Dbuf[(int64_t)head * p.T + s0 + qrow] : 0.f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  const int32_t kv_end = min(q0 + kBQ, L);
  const int32_t nkv = (kv_end + kBNq - 1) / kBNq;
  const int32_t wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;
  const int gi = l & 15;
  const int dsub = 16 * ((l >> 4) & 1);

  for (int32_t j = 0; j < nkv; ++j) {
    const int32_t kb = j * kBNq;
    __syncthreads();
    constexpr int CH = D / 8;
#pragma unroll
    for (int c = tid; c < kBNq * CH; c += kThreads) {
      const int r = c / CH, cc = c % CH;
      const int32_t key = kb + r;
      bf16x8 kv = {}, vv = {};
      if (key < L) {
        kv = *reinterpret_cast<const bf16x8*>(Kp + (int64_t)key * p.sk + cc * 8);
        vv = *reinterpret_cast<const bf16x8*>(Vp + (int64_t)key * p.sv + cc * 8);
      }
      *reinterpret_cast<bf16x8*>(&Ks[r * S + cc * 8]) = kv;
      *reinterpret_cast<bf16x8*>(&Vs[r * S + cc * 8]) = vv;
    }
    __syncthreads();
    if (kb > wq_hi) continue;

    f32x16 s[2], dp[2];
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      s[n2] = f32x16{};
      dp[n2] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&Ks[(32 * n2 + lq) * S + 16 * kk + 8 * h]);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Vs[(32 * n2 + lq) * S + 16 * kk + 8 * h]);
        s[n2] = mfma32(ak, qf[kk], s[n2]);
        dp[n2] = mfma32(av, df[kk], dp[n2]);
      }
    }
    const bool need_mask = (kb + kBNq - 1 > wq_lo) || (kb + kBNq > L);
    bf16x8 dsb[4];
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pr = fast_exp2(s[n2][i] * p.scale_log2 - lse2);
        if (need_mask) {
          const int32_t key = kb + 32 * n2 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key > qrow || key >= L) pr = 0.f;
        }
        const float ds = pr * (dp[n2][i] - Drow);
        dsb[2 * n2 + (i >> 3)][i & 7] = (bf16)ds;
      }
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int col = 32 * dt + dsub + 4 * (gi & 3);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16* p0 = &Ks[(16 * ks + 4 * h + (gi >> 2)) * S + col];
        const bf16x8 a = tr_read8(p0, p0 + 8 * S);
        acc[dt] = mfma32(a, dsb[ks], acc[dt]);
      }
    }
  }

  if (qvalid) {
    float* Qd = p.dq + ((int64_t)(s0 + qrow) * p.hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[dt][4 * g4 + e] * p.scale;
        *reinterpret_cast<f32x4*>(Qd + 32 * dt + 8 * g4 + 4 * h) = v4;
      }
    }
  }
}

// ------------------------------------------------------------------ dK, dV
template <int D>
__global__ void __launch_bounds__(kThreads, 1) k_bwd_dkdv(BwdParams p) {
  constexpr int S = KSt<D>::S;
  __shared__ __attribute__((aligned(16))) bf16 Qs[kBMk * S];
  __shared__ __attribute__((aligned(16))) bf16 dOs[kBMk * S];
  __shared__ float lse_s[kBMk];
  __shared__ float D_s[kBMk];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;
  const uint32_t item = blockIdx.x / (uint32_t)p.hkv, kvh = blockIdx.x % (uint32_t)p.hkv;
  if ((int32_t)item >= *p.n_items) return;
  const int32_t seg = p.items[2 * item], tile = p.items[2 * item + 1];
  const int32_t s0 = min(max(p.cu[seg], 0), (int32_t)p.T);
  const int32_t L = min(max(p.cu[seg + 1], s0), (int32_t)p.T) - s0;
  const int32_t kb = tile * kBKV;
  if (kb >= L) return;
  const int32_t key = kb + 32 * w + lq;  // this lane's key (S layout: lane <-> key)
  const bool kvalid = key < L;
  const int32_t wk_lo = kb + 32 * w;

  bf16x8 kf[D / 16], vf[D / 16];
  {
    const bf16* Kr = p.k + (int64_t)(s0 + key) * p.sk + (int64_t)kvh * D;
    const bf16* Vr = p.v + (int64_t)(s0 + key) * p.sv + (int64_t)kvh * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kf[kk] = kvalid ? *reinterpret_cast<const bf16x8*>(Kr + 16 * kk + 8 * h) : bf16x8{};
      vf[kk] = kvalid ? *reinterpret_cast<const bf16x8*>(Vr + 16 * kk + 8 * h) : bf16x8{};
    }
  }
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dka[dt] = f32x16{};
    dva[dt] = f32x16{};
  }
  const int gi = l & 15;
  const int dsub = 16 * ((l >> 4) & 1);
  const int32_t nqb = (L - kb + kBMk - 1) / kBMk;

  for (int32_t hh = 0; hh < p.group; ++hh) {
    const int32_t head = kvh * p.group + hh;
    const bf16* Qp = p.q + (int64_t)s0 * p.sq + (int64_t)head * D;
    const bf16* Op = p.dout + (int64_t)s0 * p.sdo + (int64_t)head * D;
    const float* lse_h = p.lse + (int64_t)head * p.T + s0;
    const float* D_h = p.Dbuf + (int64_t)head * p.T + s0;
    for (int32_t qb = 0; qb < nqb; ++qb) {
      const int32_t qs = kb + qb * kBMk;
      __syncthreads();
      constexpr int CH = D / 8;
#pragma unroll
      for (int c = tid; c < kBMk * CH; c += kThreads) {
        const int r = c / CH, cc = c % CH;
        const int32_t qi = qs + r;
        bf16x8 a = {}, bb = {};
        if (qi < L) {
          a = *reinterpret_cast<const bf16x8*>(Qp + (int64_t)qi * p.sq + cc * 8);
          bb = *reinterpret_cast<const bf16x8*>(Op + (int64_t)qi * p.sdo + cc * 8);
        }
        *reinterpret_cast<bf16x8*>(&Qs[r * S + cc * 8]) = a;
        *reinterpret_cast<bf16x8*>(&dOs[r * S + cc * 8]) = bb;
      }
      if (tid < kBMk) {
        const int32_t qi = qs + tid;
        lse_s[tid] = qi < L ? lse_h[qi] * kLog2e : 0.f;
        D_s[tid] = qi < L ? D_h[qi] : 0.f;
      }
      __syncthreads();
      if (qs + kBMk - 1 < wk_lo) continue;  // every query of the block precedes every key of this wave

#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
        const int32_t qm = qs + 32 * mq;
        if (qm + 31 < wk_lo) continue;
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&Qs[(32 * mq + lq) * S + 16 * kk + 8 * h]);
          const bf16x8 ad = *reinterpret_cast<const bf16x8*>(&dOs[(32 * mq + lq) * S + 16 * kk + 8 * h]);
          s = mfma32(aq, kf[kk], s);
          dp = mfma32(ad, vf[kk], dp);
        }
        // s[i], dp[i] <-> query 32*mq + 8*(i/4) + 4*h + i%4 of the block, key = this lane's key
        const bool need_mask = (qm < wk_lo + 31) || (qm + 32 > L);
        bf16x8 pa[2], da[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = 32 * mq + 8 * (i >> 2) + 4 * h + (i & 3);
          float pr = fast_exp2(s[i] * p.scale_log2 - lse_s[qi]);
          if (need_mask) {
            const int32_t qa = qs + qi;
            if (qa < key || qa >= L) pr = 0.f;
          }
          const float ds = pr * (dp[i] - D_s[qi]);
          pa[i >> 3][i & 7] = (bf16)pr;
          da[i >> 3][i & 7] = (bf16)ds;
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int col = 32 * dt + dsub + 4 * (gi & 3);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int row = 32 * mq + 16 * ks + 4 * h + (gi >> 2);
            const bf16* po = &dOs[row * S + col];
            const bf16* pq = &Qs[row * S + col];
            const bf16x8 bo = tr_read8(po, po + 8 * S);
            const bf16x8 bq = tr_read8(pq, pq + 8 * S);
            dva[dt] = mfma32(pa[ks], bo, dva[dt]);
            dka[dt] = mfma32(da[ks], bq, dka[dt]);
          }
        }
      }
    }
  }

  // dka/dva C layout: key = kb + 32*w + 8*(i/4) + 4*h + i%4, d = 32*dt + lq
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int32_t kr = wk_lo + 8 * (i >> 2) + 4 * h + (i & 3);
    if (kr < L) {
      float* dkr = p.dk + ((int64_t)(s0 + kr) * p.hkv + kvh) * D;
      float* dvr = p.dv + ((int64_t)(s0 + kr) * p.hkv + kvh) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        dkr[32 * dt + lq] = dka[dt][i] * p.scale;
        dvr[32 * dt + lq] = dva[dt][i];
      }
    }
  }
}

}  // namespace

static size_t dbuf_bytes(const AttnDims& d) { return align_up(sizeof(float) * (size_t)d.hq * d.T, 256); }

size_t attn_bwd_workspace_bytes(int dtype, const AttnDims& d) {
  if (dtype != 1) return dbuf_bytes(d);
  return dbuf_bytes(d) + schedule_bytes(d.T, d.n_seg, d.max_seqlen, kBQ, kBNq) +
         schedule_bytes(d.T, d.n_seg, d.max_seqlen, kBKV, kBMk);
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  const AttnDims& d = a.dims;
  char* ws = static_cast<char*>(a.workspace);
  float* Dbuf = reinterpret_cast<float*>(ws);
  ws += dbuf_bytes(d);
  TileSchedule sq = schedule_carve(ws, d.T, d.n_seg, d.max_seqlen, kBQ, kBNq);
  ws += schedule_bytes(d.T, d.n_seg, d.max_seqlen, kBQ, kBNq);
  TileSchedule sk = schedule_carve(ws, d.T, d.n_seg, d.max_seqlen, kBKV, kBMk);

  BwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.o = static_cast<const bf16*>(a.o);
  p.dout = static_cast<const bf16*>(a.dout);
  p.lse = a.lse;
  p.Dbuf = Dbuf;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  p.sdo = a.sdo;
  p.T = d.T;
  p.cu = a.cu;
  p.hq = d.hq;
  p.hkv = d.hkv;
  p.group = d.hq / d.hkv;
  p.scale = d.scale;
  p.scale_log2 = d.scale * kLog2e;
  if (d.T == 0) return hipSuccess;

  const int64_t pre_threads = d.T * d.hq * (d.d / 8);
  const unsigned pre_grid = (unsigned)((pre_threads + kThreads - 1) / kThreads);
  {
    ScopedKernelTimer timed(kTimeBwdPre, stream);
    if (d.d == 128)
      k_bwd_pre<128><<<pre_grid, kThreads, 0, stream>>>(p);
    else
      k_bwd_pre<64><<<pre_grid, kThreads, 0, stream>>>(p);
  }

  hipError_t e = launch_schedule(a.cu, d.n_seg, (int32_t)d.T, kBKV, kBMk, true, sk, stream);
  if (e != hipSuccess) return e;
  p.items = sk.items;
  p.n_items = sk.n_items;
  const unsigned grid_kv = (unsigned)(sk.cap * d.hkv);
  {
    ScopedKernelTimer timed(kTimeBwdDkdv, stream);
    if (d.d == 128)
      k_bwd_dkdv<128><<<grid_kv, kThreads, 0, stream>>>(p);
    else
      k_bwd_dkdv<64><<<grid_kv, kThreads, 0, stream>>>(p);
  }

  e = launch_schedule(a.cu, d.n_seg, (int32_t)d.T, kBQ, kBNq, false, sq, stream);
  if (e != hipSuccess) return e;
  p.items = sq.items;
  p.n_items = sq.n_items;
  const unsigned grid_q = (unsigned)(sq.cap * d.hq);
  {
    ScopedKernelTimer timed(kTimeBwdDq, stream);
    if (d.d == 128)
      k_bwd_dq<128><<<grid_q, kThreads, 0, stream>>>(p);
    else
      k_bwd_dq<64><<<grid_q, kThreads, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace psc

// Document-causal attention forward, bf16 in / fp32 accumulate, gfx950.
//
// One workgroup = one (query tile of 128 rows inside one document, query
// head).  Four waves own 32 query rows each.  The key/value loop runs over
// 64-key blocks from the document start to the tile's last row, so only tiles
// inside the document's causal triangle are visited and no mask is stored
// ("Sample Packing：长序列 LLM 训练的 Attention 问题及优化", sections 三 and 5.1).
//
// Per 64-key block and wave (layouts in attn_common.h):
//   S^T = K Q^T    A = K rows from LDS, B = Q kept in registers; each lane
//                  then holds 32 scores of its own query row.
//   online softmax in the exp2 domain (scale*log2(e) folded in), fp32 running
//                  max (shared by the two lane halves) and per-lane partial sum.
//   O^T += V^T P^T A = V read column-wise from LDS with ds_read_b64_tr_b16,
//                  B = P rounded to bf16 straight from the score registers.
// Epilogue: O / l in bf16, lse = (m + log2 l) * ln 2 in fp32.
#include "attn_common.h"
#include "psc_internal.h"

namespace psc {
namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per block
constexpr int kThreads = 256;

template <int D>
struct FwdLds {
  static constexpr int KS = D + 8;   // K row stride (elements)
  static constexpr int VS = D + 16;  // V row stride (elements)
};

struct FwdParams {
  const bf16 *q, *k, *v;
  bf16* out;
  float* lse;
  int64_t sq, sk, sv, so, T;
  const int32_t* cu;
  const int32_t* items;
  const int32_t* n_items;
  int32_t hq, group;
  float scale_log2;
};

template <int D>
__global__ void __launch_bounds__(kThreads, 2) k_attn_fwd(FwdParams p) {
  using L_ = FwdLds<D>;
  __shared__ __attribute__((aligned(16))) bf16 Ks[kBN * L_::KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kBN * L_::VS];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, lq = l & 31;
  const uint32_t b = xcd_group_remap(blockIdx.x, gridDim.x, (uint32_t)p.group);
  const uint32_t item = b / (uint32_t)p.hq, head = b % (uint32_t)p.hq;
  if ((int32_t)item >= *p.n_items) return;
  const int32_t seg = p.items[2 * item], tile = p.items[2 * item + 1];
  // segment bounds clamped to [0, T]: a malformed cu_seqlens cannot send any
  // access outside the tensors
  const int32_t s0 = min(max(p.cu[seg], 0), (int32_t)p.T);
  const int32_t L = min(max(p.cu[seg + 1], s0), (int32_t)p.T) - s0;
  const int32_t q0 = tile * kBM;
  if (q0 >= L) return;
  const int32_t kvh = (int32_t)head / p.group;

  const bf16* Qp = p.q + (int64_t)s0 * p.sq + (int64_t)head * D;
  const bf16* Kp = p.k + (int64_t)s0 * p.sk + (int64_t)kvh * D;
  const bf16* Vp = p.v + (int64_t)s0 * p.sv + (int64_t)kvh * D;

  const int32_t qrow = q0 + 32 * w + lq;
  const bool qvalid = qrow < L;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = qvalid ? *reinterpret_cast<const bf16x8*>(Qp + (int64_t)qrow * p.sq + 16 * kk + 8 * h)
                    : bf16x8{};
  }

  float m_i = -INFINITY, l_i = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};

  const int32_t kv_end = min(q0 + kBM, L);
  const int32_t nkv = (kv_end + kBN - 1) / kBN;
  const int32_t wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;
  const int gi = l & 15;
  const int dsub = 16 * ((l >> 4) & 1);

  for (int32_t j = 0; j < nkv; ++j) {
    const int32_t kb = j * kBN;
    __syncthreads();
    constexpr int CH = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int c = tid; c < kBN * CH; c += kThreads) {
      const int r = c / CH, cc = c % CH;
      const int32_t key = kb + r;
      bf16x8 kv = {}, vv = {};
      if (key < L) {
        kv = *reinterpret_cast<const bf16x8*>(Kp + (int64_t)key * p.sk + cc * 8);
        vv = *reinterpret_cast<const bf16x8*>(Vp + (int64_t)key * p.sv + cc * 8);
      }
      *reinterpret_cast<bf16x8*>(&Ks[r * L_::KS + cc * 8]) = kv;
      *reinterpret_cast<bf16x8*>(&Vs[r * L_::VS + cc * 8]) = vv;
    }
    __syncthreads();
    if (kb > wq_hi) continue;  // block entirely above this wave's rows

    f32x16 s[2];
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      s[n2] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(32 * n2 + lq) * L_::KS + 16 * kk + 8 * h]);
        s[n2] = mfma32(a, qf[kk], s[n2]);
      }
    }

    const bool need_mask = (kb + kBN - 1 > wq_lo) || (kb + kBN > L);
    float mx = -INFINITY;
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[n2][i] * p.scale_log2;
        if (need_mask) {
          const int32_t key = kb + 32 * n2 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key > qrow || key >= L) x = -INFINITY;
        }
        s[n2][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = max_halves(mx);
    const float m_new = fmaxf(m_i, mx);
    const float alpha = fast_exp2(m_i - m_new);
    float rs = 0.f;
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(s[n2][i] - m_new);
        s[n2][i] = e;
        rs += e;
      }
    }
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;

    bf16x8 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pb[ks][jj] = (bf16)s[ks >> 1][8 * (ks & 1) + jj];
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int col = 32 * dt + dsub + 4 * (gi & 3);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16* p0 = &Vs[(16 * ks + 4 * h + (gi >> 2)) * L_::VS + col];
        const bf16x8 a = tr_read8(p0, p0 + 8 * L_::VS);
        oacc[dt] = mfma32(a, pb[ks], oacc[dt]);
      }
    }
  }

  const float lt = sum_halves(l_i);
  if (qvalid) {
    const float inv = 1.f / lt;
    bf16* Op = p.out + (int64_t)(s0 + qrow) * p.so + (int64_t)head * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (bf16)(oacc[dt][4 * g4 + e] * inv);
        *reinterpret_cast<bf16x4*>(Op + 32 * dt + 8 * g4 + 4 * h) = o4;
      }
    }
    if (h == 0) p.lse[(int64_t)head * p.T + s0 + qrow] = (m_i + __log2f(lt)) * kLn2;
  }
}

}  // namespace

size_t attn_fwd_workspace_bytes(int dtype, const AttnDims& d) {
  if (dtype != 1) return 256;
  return schedule_bytes(d.T, d.n_seg, d.max_seqlen, kBM, kBN);
}

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a, hipStream_t stream) {
  const AttnDims& d = a.dims;
  TileSchedule s = schedule_carve(a.workspace, d.T, d.n_seg, d.max_seqlen, kBM, kBN);
  hipError_t e = launch_schedule(a.cu, d.n_seg, (int32_t)d.T, kBM, kBN, false, s, stream);
  if (e != hipSuccess) return e;
  FwdParams p;
  p.q = static_cast<const bf16*>(a.q);
  p.k = static_cast<const bf16*>(a.k);
  p.v = static_cast<const bf16*>(a.v);
  p.out = static_cast<bf16*>(a.out);
  p.lse = a.lse;
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  p.T = d.T;
  p.cu = a.cu;
  p.items = s.items;
  p.n_items = s.n_items;
  p.hq = d.hq;
  p.group = d.hq / d.hkv;
  p.scale_log2 = d.scale * kLog2e;
  const uint64_t grid = (uint64_t)s.cap * (uint64_t)d.hq;
  if (grid == 0) return hipSuccess;
  ScopedKernelTimer timed(kTimeFwd, stream);
  if (d.d == 128)
    k_attn_fwd<128><<<(unsigned)grid, kThreads, 0, stream>>>(p);
  else
    k_attn_fwd<64><<<(unsigned)grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace psc

// C ABI of libpsc.so (declared in include/psc.h): argument checks, sizing,
// workspace carving and launches on the caller's stream.  Every check runs on
// the host before anything is enqueued; no HIP call is made on an error path.
#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "../../include/psc.h"
#include "psc_internal.h"

namespace {

constexpr int64_t kMaxPacked = int64_t(1) << 30;
constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();

int pack_dims(int mode, int64_t n_docs, int64_t n_tokens, int32_t micro_bsz, int32_t seq_len,
              int64_t* n_rows, int64_t* max_segments) {
  if (mode != PSC_BUILD_PACK && mode != PSC_BUILD_UNPACK) return PSC_ERR_INVALID;
  if (n_docs < 0 || n_tokens < 0 || micro_bsz < 1 || seq_len < 1) return PSC_ERR_INVALID;
  const int64_t PL = (int64_t)micro_bsz * seq_len;
  if (PL > kMaxPacked) return PSC_ERR_INVALID;
  if (n_docs >= kI32Max || n_tokens >= kI32Max) return PSC_ERR_INVALID;
  const int64_t rows = mode == PSC_BUILD_PACK ? (n_tokens + PL - 1) / PL : (n_docs + micro_bsz - 1) / micro_bsz;
  if (rows * PL > kI32Max) return PSC_ERR_INVALID;  // cu_seqlens is int32
  const int64_t segs = mode == PSC_BUILD_PACK ? n_docs + 2 * rows : n_docs + rows;
  if (segs >= kI32Max) return PSC_ERR_INVALID;
  *n_rows = rows;
  *max_segments = segs;
  return PSC_OK;
}

bool supported_head_dim(int32_t d) { return d == 32 || d == 64 || d == 128; }

int attn_dims(int dtype, int64_t T, int32_t n_seg, int32_t max_seqlen, int32_t hq, int32_t hkv, int32_t head_dim,
              float softmax_scale, psc::AttnDims* out) {
  if (dtype != PSC_F32 && dtype != PSC_BF16) return PSC_ERR_INVALID;
  if (T < 0 || T > kI32Max || n_seg < 0 || hq < 1 || hkv < 1 || head_dim < 1) return PSC_ERR_INVALID;
  if (hq % hkv != 0) return PSC_ERR_INVALID;
  if (T > 0 && (n_seg < 1 || n_seg > T || max_seqlen < 1 || max_seqlen > T)) return PSC_ERR_INVALID;
  if (!supported_head_dim(head_dim)) return PSC_ERR_UNSUPPORTED;
  if (!(softmax_scale == softmax_scale) || std::isinf(softmax_scale)) return PSC_ERR_INVALID;
  out->T = T;
  out->n_seg = n_seg;
  out->max_seqlen = max_seqlen < 1 ? 1 : max_seqlen;
  out->hq = hq;
  out->hkv = hkv;
  out->d = head_dim;
  out->scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  return PSC_OK;
}

// Token stride and base alignment of one [T, heads, D] operand.
bool operand_ok(const void* p, int64_t tok_stride, int32_t heads, int32_t d, int dtype, int64_t T) {
  if (T == 0) return true;
  if (!p) return false;
  if (tok_stride < (int64_t)heads * d) return false;
  if (dtype == PSC_BF16) {
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return false;
    if ((tok_stride * 2) % 16 != 0) return false;
    // the bf16 kernels address a 64-row tile with 32-bit byte offsets
    if (tok_stride > ((int64_t)1 << 25)) return false;
  } else {
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0) return false;
  }
  return true;
}

// Debug builds (PSC_DEBUG_CHECKS) keep 256 bytes at the end of the attention
// workspaces for the cu_seqlens check's flags word.
#ifdef PSC_DEBUG_CHECKS
constexpr size_t kDebugTail = 256;
#else
constexpr size_t kDebugTail = 0;
#endif

// (cos, sin) table of the in-kernel rotary turns: positions [0, max_seqlen)
// x head_dim / 2 frequencies, float2 each.
size_t rope_table_bytes(const psc::AttnDims& d) {
  return psc::align_up((size_t)d.max_seqlen * (size_t)(d.d / 2) * sizeof(float2), 256);
}

// Workspace of pass 0 (fwd), 1 (bwd), 2 (fwd with rotary turns), 3 (bwd with
// rotary turns): the kernels' scratch, then the turn table (passes 2, 3),
// then the debug flags word.
size_t attn_part(int pass, int dtype, const psc::AttnDims& d) {
  return pass % 2 == 0 ? psc::attn_fwd_workspace_bytes(dtype, d) : psc::attn_bwd_workspace_bytes(dtype, d);
}
// A caller's workspace: PSC_ERR_WORKSPACE when missing or shorter than
// `need`, PSC_ERR_INVALID when not 16-byte aligned (the kernels read the
// schedule entries carved from it as 16-byte vectors).
int workspace_status(const void* ws, size_t bytes, size_t need) {
  if (!ws || bytes < need) return PSC_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return PSC_ERR_INVALID;
  return PSC_OK;
}

size_t workspace_for(int pass, int dtype, const psc::AttnDims& d) {
  return attn_part(pass, dtype, d) + (pass >= 2 ? rope_table_bytes(d) : 0) + kDebugTail;
}

// Checks of the rotary arguments of the fused entry points (host only).
int rope_checks(int dtype, int32_t head_dim, const int32_t* positions, float base, int64_t T) {
  if (!(base > 0.f) || std::isinf(base)) return PSC_ERR_INVALID;
  if (T > 0 && !positions) return PSC_ERR_INVALID;
  if (dtype != PSC_BF16 || (head_dim != 64 && head_dim != 128)) return PSC_ERR_UNSUPPORTED;
  return PSC_OK;
}

psc::RopeArgs rope_args(int dtype, int32_t head_dim, float base) {
  psc::RopeArgs a{};
  a.dtype = dtype;
  a.d = head_dim;
  for (int i = 0; i < 64; ++i)
    a.inv_freq[i] = i < head_dim / 2 ? std::pow((double)base, -2.0 * i / head_dim) : 0.0;
  return a;
}

#ifdef PSC_DEBUG_CHECKS
// Runs the cu_seqlens check on `stream`, waits for it and maps the flags to a
// status (the one synchronising path of the library; debug builds only).
int debug_check_cu(const int32_t* cu, int32_t n_seg, int64_t T, void* ws, size_t need, hipStream_t stream) {
  int32_t* flags = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + need - kDebugTail);
  if (psc::launch_check_cu(cu, n_seg, (int32_t)T, flags, stream) != hipSuccess) return PSC_ERR_HIP;
  int32_t h = 0;
  if (hipMemcpyAsync(&h, flags, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess) return PSC_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return PSC_ERR_HIP;
  return psc_cu_seqlens_status(h);
}
#endif

// Argument checks of the forward (both entry points), host only.
int fwd_checks(int dtype, const void* q, const void* k, const void* v, int64_t q_tok_stride, int64_t k_tok_stride,
               int64_t v_tok_stride, const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
               int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim, float softmax_scale,
               const void* out, int64_t out_tok_stride, const float* lse, psc::AttnDims* d) {
  int st = attn_dims(dtype, total_tokens, n_segments, max_seqlen, hq, hkv, head_dim, softmax_scale, d);
  if (st != PSC_OK) return st;
  const int64_t T = total_tokens;
  if (!operand_ok(q, q_tok_stride, hq, head_dim, dtype, T) || !operand_ok(k, k_tok_stride, hkv, head_dim, dtype, T) ||
      !operand_ok(v, v_tok_stride, hkv, head_dim, dtype, T) ||
      !operand_ok(out, out_tok_stride, hq, head_dim, dtype, T))
    return PSC_ERR_INVALID;
  if (T > 0 && (!cu_seqlens || !lse)) return PSC_ERR_INVALID;
  return PSC_OK;
}

// Launch of a checked forward with a workspace of at least `need` bytes.
int fwd_launch(int dtype, const psc::AttnDims& d, const void* q, const void* k, const void* v, int64_t sq, int64_t sk,
               int64_t sv, const int32_t* cu_seqlens, void* out, int64_t so, float* lse, void* workspace, size_t need,
               hipStream_t stream, const psc::AttnRope& rope = psc::AttnRope()) {
#ifdef PSC_DEBUG_CHECKS
  // need == 0: the caller ran the check before its own launches
  if (need > 0)
    if (int c = debug_check_cu(cu_seqlens, d.n_seg, d.T, workspace, need, stream)) return c;
#else
  (void)need;
#endif
  psc::AttnFwdArgs a;
  a.dims = d;
  a.q = q;
  a.k = k;
  a.v = v;
  a.sq = sq;
  a.sk = sk;
  a.sv = sv;
  a.so = so;
  a.cu = cu_seqlens;
  a.out = out;
  a.lse = lse;
  a.workspace = workspace;
  a.rope = rope;
  hipError_t e = dtype == PSC_BF16 ? psc::launch_attn_fwd_bf16(a, stream) : psc::launch_attn_fwd_f32(a, stream);
  return e == hipSuccess ? PSC_OK : PSC_ERR_HIP;
}

// Argument checks of the backward (both entry points), host only.
int bwd_checks(int dtype, int grad_dtype, const void* q, const void* k, const void* v, const void* out,
               const void* dout, const float* lse, int64_t sq, int64_t sk, int64_t sv, int64_t so, int64_t sdo,
               const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen, int64_t total_tokens, int32_t hq,
               int32_t hkv, int32_t head_dim, float softmax_scale, const void* dq, const void* dk, const void* dv,
               psc::AttnDims* d) {
  int st = attn_dims(dtype, total_tokens, n_segments, max_seqlen, hq, hkv, head_dim, softmax_scale, d);
  if (st != PSC_OK) return st;
  if (grad_dtype != PSC_F32 && grad_dtype != PSC_BF16) return PSC_ERR_INVALID;
  if (dtype == PSC_F32 && grad_dtype != PSC_F32) return PSC_ERR_UNSUPPORTED;
  const int64_t T = total_tokens;
  if (!operand_ok(q, sq, hq, head_dim, dtype, T) || !operand_ok(k, sk, hkv, head_dim, dtype, T) ||
      !operand_ok(v, sv, hkv, head_dim, dtype, T) || !operand_ok(out, so, hq, head_dim, dtype, T) ||
      !operand_ok(dout, sdo, hq, head_dim, dtype, T))
    return PSC_ERR_INVALID;
  if (T > 0 && (!cu_seqlens || !lse || !dq || !dk || !dv)) return PSC_ERR_INVALID;
  if (T > 0 && ((reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk) |
                 reinterpret_cast<uintptr_t>(dv)) % 16 != 0))
    return PSC_ERR_INVALID;
  return PSC_OK;
}

int bwd_launch(int dtype, int grad_dtype, const psc::AttnDims& d, const void* q, const void* k, const void* v,
               const void* out, const void* dout, const float* lse, int64_t sq, int64_t sk, int64_t sv, int64_t so,
               int64_t sdo, const int32_t* cu_seqlens, void* dq, void* dk, void* dv, void* workspace, size_t need,
               hipStream_t stream, const psc::AttnRope& rope = psc::AttnRope()) {
#ifdef PSC_DEBUG_CHECKS
  // need == 0: the caller ran the check before its own launches
  if (need > 0)
    if (int c = debug_check_cu(cu_seqlens, d.n_seg, d.T, workspace, need, stream)) return c;
#else
  (void)need;
#endif
  psc::AttnBwdArgs a;
  a.dims = d;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.dout = dout;
  a.lse = lse;
  a.sq = sq;
  a.sk = sk;
  a.sv = sv;
  a.so = so;
  a.sdo = sdo;
  a.cu = cu_seqlens;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.grad_bf16 = grad_dtype == PSC_BF16;
  a.workspace = workspace;
  a.rope = rope;
  hipError_t e = dtype == PSC_BF16 ? psc::launch_attn_bwd_bf16(a, stream) : psc::launch_attn_bwd_f32(a, stream);
  return e == hipSuccess ? PSC_OK : PSC_ERR_HIP;
}

// ------------------------------------------------- allocation-free forward
//
// psc_varlen_attn_fwd_noalloc keeps its workspace (the tile schedule) in this
// file-scope device array instead of a caller buffer.  Each GPU the library
// runs on holds its own copy, at its own address, until the process ends.  On
// the host `scratch` names a host-side stand-in, never the device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is passed to kernels.  Nothing in
// it has to start at zero: the schedule kernel clears its own histogram and
// writes every entry the attention kernel reads.  All calls on one GPU share
// the array, so calls that overlap in time on one GPU race.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream`.
int scratch_for(hipStream_t stream, void** out) {
  int dev = 0, cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return PSC_ERR_HIP;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return PSC_ERR_HIP;
  } else {
    dev = cur;
  }
  if (dev < 0 || dev >= kMaxDevices) return PSC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return PSC_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return PSC_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PSC_OK;
}

}  // namespace

extern "C" {

const char* psc_strerror(int status) {
  switch (status) {
    case PSC_OK: return "ok";
    case PSC_ERR_INVALID: return "invalid argument";
    case PSC_ERR_UNSUPPORTED: return "unsupported configuration";
    case PSC_ERR_WORKSPACE: return "workspace missing or too small";
    case PSC_ERR_CAPACITY: return "output capacity too small";
    case PSC_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int psc_version(void) { return 100; }

int psc_pack_sizes(int mode, int64_t n_docs, int64_t n_tokens, int32_t micro_bsz, int32_t seq_len,
                   int64_t* n_rows, int64_t* max_segments, size_t* workspace_bytes) {
  if (!n_rows || !max_segments || !workspace_bytes) return PSC_ERR_INVALID;
  int64_t rows, segs;
  int st = pack_dims(mode, n_docs, n_tokens, micro_bsz, seq_len, &rows, &segs);
  if (st != PSC_OK) return st;
  *n_rows = rows;
  *max_segments = segs;
  *workspace_bytes = psc::pack_workspace_bytes(n_docs, rows);
  return PSC_OK;
}

int psc_pack_build(int mode, const int32_t* tokens, const int64_t* doc_offsets, int64_t n_docs, int64_t n_tokens,
                   int32_t micro_bsz, int32_t seq_len, int64_t n_rows, int32_t* input_ids, int32_t* labels,
                   int32_t* indexes, int32_t* cu_seqlens, int64_t max_segments, int32_t* row_seg_ptr,
                   int32_t* row_valid_len, int32_t* stats, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int64_t rows, segs;
  int st = pack_dims(mode, n_docs, n_tokens, micro_bsz, seq_len, &rows, &segs);
  if (st != PSC_OK) return st;
  if (n_rows != rows) return PSC_ERR_INVALID;
  if (!doc_offsets || !cu_seqlens || !row_seg_ptr || !stats) return PSC_ERR_INVALID;
  if (n_tokens > 0 && !tokens) return PSC_ERR_INVALID;
  if (rows > 0 && (!input_ids || !labels || !indexes)) return PSC_ERR_INVALID;
  if (n_docs == 0 && n_tokens != 0) return PSC_ERR_INVALID;
  if (max_segments < segs) return PSC_ERR_CAPACITY;
  const size_t need = psc::pack_workspace_bytes(n_docs, rows);
  if (int c = workspace_status(workspace, workspace_bytes, need)) return c;

  psc::PackArgs a;
  a.mode = mode;
  a.tokens = tokens;
  a.doc_offsets = doc_offsets;
  a.n_docs = n_docs;
  a.n_tokens = n_tokens;
  a.micro_bsz = micro_bsz;
  a.seq_len = seq_len;
  a.packed_length = micro_bsz * seq_len;
  a.n_rows = rows;
  a.input_ids = input_ids;
  a.labels = labels;
  a.indexes = indexes;
  a.cu_seqlens = cu_seqlens;
  a.row_seg_ptr = row_seg_ptr;
  a.row_valid_len = row_valid_len;
  a.stats = stats;
  a.max_segments = max_segments;
  a.workspace = workspace;
  return psc::launch_pack(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PSC_OK : PSC_ERR_HIP;
}

int psc_varlen_attn_workspace(int pass, int dtype, int64_t total_tokens, int32_t n_segments, int32_t max_seqlen,
                              int32_t hq, int32_t hkv, int32_t head_dim, size_t* bytes) {
  if (!bytes || pass < 0 || pass > 3) return PSC_ERR_INVALID;
  psc::AttnDims d;
  int st = attn_dims(dtype, total_tokens, n_segments, max_seqlen, hq, hkv, head_dim, 0.f, &d);
  if (st != PSC_OK) return st;
  *bytes = workspace_for(pass, dtype, d);
  return PSC_OK;
}

int psc_varlen_attn_fwd(int dtype, const void* q, const void* k, const void* v, int64_t q_tok_stride,
                        int64_t k_tok_stride, int64_t v_tok_stride, const int32_t* cu_seqlens, int32_t n_segments,
                        int32_t max_seqlen, int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                        float softmax_scale, void* out, int64_t out_tok_stride, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  psc::AttnDims d;
  int st = fwd_checks(dtype, q, k, v, q_tok_stride, k_tok_stride, v_tok_stride, cu_seqlens, n_segments, max_seqlen,
                      total_tokens, hq, hkv, head_dim, softmax_scale, out, out_tok_stride, lse, &d);
  if (st != PSC_OK) return st;
  const int64_t T = total_tokens;
  const size_t need = workspace_for(0, dtype, d);
  if (T > 0)
    if (int c = workspace_status(workspace, workspace_bytes, need)) return c;
  if (T == 0) return PSC_OK;
  return fwd_launch(dtype, d, q, k, v, q_tok_stride, k_tok_stride, v_tok_stride, cu_seqlens, out, out_tok_stride,
                    lse, workspace, need, static_cast<hipStream_t>(stream));
}

int psc_varlen_attn_fwd_noalloc(int dtype, const void* q, const void* k, const void* v, int64_t q_tok_stride,
                                int64_t k_tok_stride, int64_t v_tok_stride, const int32_t* cu_seqlens,
                                int32_t n_segments, int32_t max_seqlen, int64_t total_tokens, int32_t hq,
                                int32_t hkv, int32_t head_dim, float softmax_scale, void* out,
                                int64_t out_tok_stride, float* lse, void* stream) {
  psc::AttnDims d;
  int st = fwd_checks(dtype, q, k, v, q_tok_stride, k_tok_stride, v_tok_stride, cu_seqlens, n_segments, max_seqlen,
                      total_tokens, hq, hkv, head_dim, softmax_scale, out, out_tok_stride, lse, &d);
  if (st != PSC_OK) return st;
  const int64_t T = total_tokens;
  const size_t need = workspace_for(0, dtype, d);
  if (need > kScratchBytes) return PSC_ERR_WORKSPACE;  // beyond the built-in scratch
  if (T == 0) return PSC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = scratch_for(s, &ws);
  if (st != PSC_OK) return st;
  return fwd_launch(dtype, d, q, k, v, q_tok_stride, k_tok_stride, v_tok_stride, cu_seqlens, out, out_tok_stride,
                    lse, ws, need, s);
}

int psc_varlen_attn_bwd(int dtype, int grad_dtype, const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, int64_t q_tok_stride, int64_t k_tok_stride,
                        int64_t v_tok_stride, int64_t out_tok_stride, int64_t dout_tok_stride,
                        const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen, int64_t total_tokens,
                        int32_t hq, int32_t hkv, int32_t head_dim, float softmax_scale, void* dq, void* dk,
                        void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  psc::AttnDims d;
  int st = bwd_checks(dtype, grad_dtype, q, k, v, out, dout, lse, q_tok_stride, k_tok_stride, v_tok_stride,
                      out_tok_stride, dout_tok_stride, cu_seqlens, n_segments, max_seqlen, total_tokens, hq, hkv,
                      head_dim, softmax_scale, dq, dk, dv, &d);
  if (st != PSC_OK) return st;
  const size_t need = workspace_for(1, dtype, d);
  if (total_tokens > 0)
    if (int c = workspace_status(workspace, workspace_bytes, need)) return c;
  if (total_tokens == 0) return PSC_OK;
  return bwd_launch(dtype, grad_dtype, d, q, k, v, out, dout, lse, q_tok_stride, k_tok_stride, v_tok_stride,
                    out_tok_stride, dout_tok_stride, cu_seqlens, dq, dk, dv, workspace, need,
                    static_cast<hipStream_t>(stream));
}

int psc_varlen_attn_fwd_rope(int dtype, void* q, void* k, const void* v, int64_t q_tok_stride, int64_t k_tok_stride,
                             int64_t v_tok_stride, const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                             int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                             const int32_t* positions, float rope_base, float softmax_scale, void* out,
                             int64_t out_tok_stride, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  psc::AttnDims d;
  int st = fwd_checks(dtype, q, k, v, q_tok_stride, k_tok_stride, v_tok_stride, cu_seqlens, n_segments, max_seqlen,
                      total_tokens, hq, hkv, head_dim, softmax_scale, out, out_tok_stride, lse, &d);
  if (st != PSC_OK) return st;
  st = rope_checks(dtype, head_dim, positions, rope_base, total_tokens);
  if (st != PSC_OK) return st;
  const int64_t T = total_tokens;
  const size_t need = workspace_for(2, dtype, d);
  if (T > 0)
    if (int c = workspace_status(workspace, workspace_bytes, need)) return c;
  if (T == 0) return PSC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
#ifdef PSC_DEBUG_CHECKS
  if (int c = debug_check_cu(cu_seqlens, n_segments, T, workspace, need, s)) return c;
#endif
  // the turn table, then k turned in place by the rotation kernel; q is
  // turned inside the attention kernel as it is loaded, and written back
  float2* table = reinterpret_cast<float2*>(static_cast<char*>(workspace) + attn_part(2, dtype, d));
  psc::RopeArgs ra = rope_args(dtype, head_dim, rope_base);
  ra.T = T;
  ra.pos = positions;
  if (psc::launch_rope_table(ra, d.max_seqlen, table, s) != hipSuccess) return PSC_ERR_HIP;
  psc::RopeArgs rk = ra;
  rk.q = k;
  rk.sq = k_tok_stride;
  rk.hq = hkv;
  rk.k = nullptr;
  rk.sk = 0;
  rk.hkv = 0;
  rk.inverse = 0;
  if (psc::launch_rope(rk, s) != hipSuccess) return PSC_ERR_HIP;
  psc::AttnRope rope;
  rope.pos = positions;
  rope.rope_cs = table;
  rope.rope_n_pos = d.max_seqlen;
  return fwd_launch(dtype, d, q, k, v, q_tok_stride, k_tok_stride, v_tok_stride, cu_seqlens, out, out_tok_stride,
                    lse, workspace, 0, s, rope);
}

int psc_varlen_attn_bwd_rope(int dtype, int grad_dtype, const void* q_rot, const void* k_rot, const void* v,
                             const void* out, const void* dout, const float* lse, int64_t q_tok_stride,
                             int64_t k_tok_stride, int64_t v_tok_stride, int64_t out_tok_stride,
                             int64_t dout_tok_stride, const int32_t* cu_seqlens, int32_t n_segments,
                             int32_t max_seqlen, int64_t total_tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                             const int32_t* positions, float rope_base, float softmax_scale, void* dq, void* dk,
                             void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  psc::AttnDims d;
  int st = bwd_checks(dtype, grad_dtype, q_rot, k_rot, v, out, dout, lse, q_tok_stride, k_tok_stride, v_tok_stride,
                      out_tok_stride, dout_tok_stride, cu_seqlens, n_segments, max_seqlen, total_tokens, hq, hkv,
                      head_dim, softmax_scale, dq, dk, dv, &d);
  if (st != PSC_OK) return st;
  st = rope_checks(dtype, head_dim, positions, rope_base, total_tokens);
  if (st != PSC_OK) return st;
  const size_t need = workspace_for(3, dtype, d);
  if (total_tokens > 0)
    if (int c = workspace_status(workspace, workspace_bytes, need)) return c;
  if (total_tokens == 0) return PSC_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
#ifdef PSC_DEBUG_CHECKS
  if (int c = debug_check_cu(cu_seqlens, n_segments, total_tokens, workspace, need, s)) return c;
#endif
  float2* table = reinterpret_cast<float2*>(static_cast<char*>(workspace) + attn_part(3, dtype, d));
  psc::RopeArgs ra = rope_args(dtype, head_dim, rope_base);
  if (psc::launch_rope_table(ra, d.max_seqlen, table, s) != hipSuccess) return PSC_ERR_HIP;
  psc::AttnRope rope;
  rope.pos = positions;
  rope.rope_cs = table;
  rope.rope_n_pos = d.max_seqlen;
  return bwd_launch(dtype, grad_dtype, d, q_rot, k_rot, v, out, dout, lse, q_tok_stride, k_tok_stride, v_tok_stride,
                    out_tok_stride, dout_tok_stride, cu_seqlens, dq, dk, dv, workspace, 0, s, rope);
}

int psc_check_cu_seqlens(const int32_t* cu_seqlens, int32_t n_segments, int64_t total_tokens, int32_t* flags,
                         void* stream) {
  if (n_segments < 0 || total_tokens < 0 || total_tokens > kI32Max) return PSC_ERR_INVALID;
  if (!cu_seqlens || !flags) return PSC_ERR_INVALID;
  const hipError_t e =
      psc::launch_check_cu(cu_seqlens, n_segments, (int32_t)total_tokens, flags, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PSC_OK : PSC_ERR_HIP;
}

int psc_cu_seqlens_status(int32_t flags) { return flags == 0 ? PSC_OK : PSC_ERR_INVALID; }

int psc_debug_checks(void) {
#ifdef PSC_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

int psc_rope(int dtype, void* q, int64_t q_tok_stride, int32_t hq, void* k, int64_t k_tok_stride, int32_t hkv,
             int64_t total_tokens, int32_t head_dim, const int32_t* positions, float base, int inverse,
             void* stream) {
  if (dtype != PSC_F32 && dtype != PSC_BF16) return PSC_ERR_INVALID;
  const int64_t T = total_tokens;
  if (T < 0 || T > kI32Max || hq < 1 || (k && hkv < 1)) return PSC_ERR_INVALID;
  if (!(base > 0.f) || std::isinf(base)) return PSC_ERR_INVALID;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return PSC_ERR_UNSUPPORTED;
  if (T == 0) return PSC_OK;
  const int64_t esize = dtype == PSC_BF16 ? 2 : 4;
  auto ok = [&](const void* p, int64_t stride, int32_t heads) {
    if (!p || stride < (int64_t)heads * head_dim) return false;
    return reinterpret_cast<uintptr_t>(p) % 16 == 0 && (stride * esize) % 16 == 0;
  };
  if (!ok(q, q_tok_stride, hq) || (k && !ok(k, k_tok_stride, hkv)) || !positions) return PSC_ERR_INVALID;
  psc::RopeArgs a;
  a.dtype = dtype;
  a.q = q;
  a.k = k;
  a.sq = q_tok_stride;
  a.sk = k ? k_tok_stride : 0;
  a.T = T;
  a.hq = hq;
  a.hkv = k ? hkv : 0;
  a.d = head_dim;
  a.inverse = inverse != 0;
  a.pos = positions;
  for (int i = 0; i < 64; ++i)
    a.inv_freq[i] = i < head_dim / 2 ? std::pow((double)base, -2.0 * i / head_dim) : 0.0;
  const hipError_t e = psc::launch_rope(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PSC_OK : PSC_ERR_HIP;
}

int psc_row_max_seqlen(const int32_t* cu_seqlens, int64_t n_cu, const int32_t* row_seg_ptr, int64_t n_rows,
                       int32_t* out, void* stream) {
  if (n_rows < 0 || n_rows >= kI32Max || n_cu < 1 || n_cu > kI32Max) return PSC_ERR_INVALID;
  if (n_rows == 0) return PSC_OK;
  if (!cu_seqlens || !row_seg_ptr || !out) return PSC_ERR_INVALID;
  const hipError_t e = psc::launch_row_max_seqlen(cu_seqlens, n_cu, row_seg_ptr, n_rows, out,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PSC_OK : PSC_ERR_HIP;
}

int psc_unpack_data(const int32_t* input_ids, const int32_t* labels, int64_t n_rows, int32_t packed_len,
                    const int32_t* cu_seqlens, int64_t n_cu, const int32_t* row_seg_ptr,
                    const int32_t* row_valid_len, int32_t micro_bsz, int32_t seq_len, int32_t* out_ids,
                    int32_t* out_labels, void* stream) {
  if (n_rows < 0 || packed_len < 1 || micro_bsz < 1 || seq_len < 1 || n_cu < 1 || n_cu > kI32Max)
    return PSC_ERR_INVALID;
  if (n_rows * (int64_t)packed_len > kI32Max) return PSC_ERR_INVALID;
  if (n_rows * (int64_t)micro_bsz * seq_len > (int64_t(1) << 40)) return PSC_ERR_INVALID;
  if (n_rows == 0) return PSC_OK;
  if (!input_ids || !labels || !cu_seqlens || !row_seg_ptr || !row_valid_len || !out_ids || !out_labels)
    return PSC_ERR_INVALID;
  psc::UnpackArgs a;
  a.input_ids = input_ids;
  a.labels = labels;
  a.cu = cu_seqlens;
  a.row_seg_ptr = row_seg_ptr;
  a.row_valid_len = row_valid_len;
  a.out_ids = out_ids;
  a.out_labels = out_labels;
  a.n_rows = n_rows;
  a.n_cu = n_cu;
  a.packed_len = packed_len;
  a.micro_bsz = micro_bsz;
  a.seq_len = seq_len;
  const hipError_t e = psc::launch_unpack(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PSC_OK : PSC_ERR_HIP;
}

int psc_split_sequence(const int32_t* in, int64_t rows, int32_t length, int32_t tp, int32_t rank, int32_t* out,
                       void* stream) {
  if (rows < 0 || length < 0 || tp < 1 || rank < 0 || rank >= tp || length % tp != 0) return PSC_ERR_INVALID;
  if (rows * (int64_t)length > (int64_t(1) << 40)) return PSC_ERR_INVALID;
  if (rows == 0 || length == 0) return PSC_OK;
  if (!in || !out) return PSC_ERR_INVALID;
  const hipError_t e = psc::launch_split(in, rows, length, tp, rank, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PSC_OK : PSC_ERR_HIP;
}

}  // extern "C"

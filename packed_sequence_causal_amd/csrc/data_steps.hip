// The data steps after the packer (InternEvo "数据加载与流程", section
// "处理数据"): packed_data_normalizer's per-row max_seqlen, unpack_data (a
// packed row back to [micro_bsz, SEQ_LEN], one document per slot) and
// split_data_sequence_parallel (one rank's slice of the sequence dimension).
// Integer gathers, one thread per output element (per row for max_seqlen);
// every read index is clamped to its row, so inconsistent boundaries cannot
// send a read outside the buffers.
#include "psc_internal.h"

namespace psc {
namespace {

constexpr int kThreads = 256;
constexpr int32_t kPadId = 0;
constexpr int32_t kIgnore = -100;

__global__ void __launch_bounds__(kThreads) k_row_max_seqlen(const int32_t* cu, int64_t n_cu, const int32_t* rsp,
                                                             int64_t n_rows, int32_t* out) {
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= n_rows) return;
  const int64_t a = min((int64_t)max(rsp[r], 0), n_cu - 1);
  const int64_t b = min((int64_t)max(rsp[r + 1], 0), n_cu - 1);
  int32_t m = 0;
  for (int64_t s = a; s < b; ++s) m = max(m, cu[s + 1] - cu[s]);
  out[r] = m;
}

// out rows o = r * micro_bsz + i hold document i of packed row r.
__global__ void __launch_bounds__(kThreads) k_unpack(UnpackArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = a.n_rows * a.micro_bsz * (int64_t)a.seq_len;
  if (gid >= total) return;
  const int64_t o = gid / a.seq_len;
  const int32_t j = (int32_t)(gid - o * a.seq_len);
  const int64_t r = o / a.micro_bsz;
  const int32_t i = (int32_t)(o - r * a.micro_bsz);
  const int64_t row0 = r * a.packed_len;
  const int64_t seg = (int64_t)max(a.row_seg_ptr[r], 0) + i;
  const int64_t seg_end = (int64_t)max(a.row_seg_ptr[r + 1], 0);
  int32_t id = kPadId, lab = kIgnore;
  if (seg < seg_end && seg + 1 < a.n_cu) {
    const int64_t s = min(max((int64_t)a.cu[seg], row0), row0 + a.packed_len);
    const int64_t e = min(max((int64_t)a.cu[seg + 1], s), row0 + a.packed_len);
    const int32_t valid = min(max(a.row_valid_len[r], 0), a.packed_len);
    // a segment that starts at or past the valid length is the padding tail
    if (s - row0 < valid && j < e - s) {
      id = a.input_ids[s + j];
      lab = a.labels[s + j];
    }
  }
  a.out_ids[gid] = id;
  a.out_labels[gid] = lab;
}

__global__ void __launch_bounds__(kThreads) k_split(const int32_t* in, int64_t rows, int32_t length, int32_t width,
                                                    int32_t rank, int32_t* out) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= rows * width) return;
  const int64_t r = gid / width;
  const int32_t j = (int32_t)(gid - r * width);
  out[gid] = in[r * length + (int64_t)rank * width + j];
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_row_max_seqlen(const int32_t* cu, int64_t n_cu, const int32_t* row_seg_ptr, int64_t n_rows,
                                 int32_t* out, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  ScopedKernelTimer timed(kTimeData, stream);
  k_row_max_seqlen<<<blocks_for(n_rows), kThreads, 0, stream>>>(cu, n_cu, row_seg_ptr, n_rows, out);
  return hipGetLastError();
}

hipError_t launch_unpack(const UnpackArgs& a, hipStream_t stream) {
  const int64_t total = a.n_rows * a.micro_bsz * (int64_t)a.seq_len;
  if (total == 0) return hipSuccess;
  ScopedKernelTimer timed(kTimeData, stream);
  k_unpack<<<blocks_for(total), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_split(const int32_t* in, int64_t rows, int32_t length, int32_t tp, int32_t rank, int32_t* out,
                        hipStream_t stream) {
  const int32_t width = length / tp;
  if (rows * width == 0) return hipSuccess;
  ScopedKernelTimer timed(kTimeData, stream);
  k_split<<<blocks_for(rows * width), kThreads, 0, stream>>>(in, rows, length, width, rank, out);
  return hipGetLastError();
}

}  // namespace psc

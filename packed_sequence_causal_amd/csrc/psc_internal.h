// Internal launch interface between the C ABI (psc_api.hip) and the kernels.
// Host-side structs only; every pointer is a device pointer.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace psc {

// Kernel timing slots (numbering matches enum psc_kernel in psc.h).
// kTimeBwdPre is kept for stable ids; nothing is timed in it.
enum TimerSlot { kTimePack = 0, kTimeSchedule, kTimeFwd, kTimeBwdPre, kTimeBwdDkdv, kTimeBwdDq, kTimeRope, kTimeData, kTimerSlots };

// Brackets the launches made during its lifetime with HIP events on `stream`
// when timing is switched on (timing.hip); does nothing otherwise.
class ScopedKernelTimer {
 public:
  ScopedKernelTimer(int slot, hipStream_t stream);
  ~ScopedKernelTimer();
  ScopedKernelTimer(const ScopedKernelTimer&) = delete;
  ScopedKernelTimer& operator=(const ScopedKernelTimer&) = delete;

 private:
  int slot_;
  hipStream_t stream_;
  void* start_ = nullptr;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- packing
struct PackArgs {
  int mode;  // 0 carry-over, 1 truncate-and-pad
  const int32_t* tokens;
  const int64_t* doc_offsets;
  int64_t n_docs, n_tokens;
  int32_t micro_bsz, seq_len, packed_length;
  int64_t n_rows;
  int32_t *input_ids, *labels, *indexes, *cu_seqlens, *row_seg_ptr, *row_valid_len, *stats;
  int64_t max_segments;
  void* workspace;
};

constexpr int kScanTile = 1024;  // items per block of the document scan

struct PackWorkspace {
  int64_t* nz_rank;     // [n_docs + 1] exclusive count of non-empty documents
  int64_t* trunc_scan;  // [n_docs + 1] exclusive sum of min(len, seq_len) over non-empty docs
  int64_t* slot_doc;    // [n_docs] index of the k-th non-empty document
  int64_t* partials;    // [2 * n_blocks] per-block sums of the scan (pairs)
  int64_t* row_aux;     // [n_rows] per-row base (see pack.hip)
  int32_t* row_valid;   // [n_rows]
  int64_t n_blocks;
};

size_t pack_workspace_bytes(int64_t n_docs, int64_t n_rows);
PackWorkspace pack_carve(void* ws, int64_t n_docs, int64_t n_rows);
hipError_t launch_pack(const PackArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- attention
struct AttnDims {
  int64_t T;
  int32_t n_seg, max_seqlen, hq, hkv, d;
  float scale;  // softmax scale (natural units)
};

// Rotary embedding inside the attention kernels (null rope_cs: none).
// rope_cs[pos * D/2 + i] = (cos, sin) of the turn of dims (i, i + D/2) at
// position pos < rope_n_pos; pos = positions[token], clamped to the table.
struct AttnRope {
  const int32_t* pos = nullptr;
  const float2* rope_cs = nullptr;
  int32_t rope_n_pos = 0;
};

struct AttnFwdArgs {
  AttnDims dims;
  const void *q, *k, *v;
  int64_t sq, sk, sv, so;  // token strides in elements
  const int32_t* cu;
  void* out;
  float* lse;
  void* workspace;
  AttnRope rope;  // with rope: q is turned in registers and written back in place
};

struct AttnBwdArgs {
  AttnDims dims;
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  int64_t sq, sk, sv, so, sdo;
  const int32_t* cu;
  void *dq, *dk, *dv;  // float32, or bf16 when grad_bf16 (bf16 inputs only)
  int32_t grad_bf16;
  void* workspace;
  AttnRope rope;  // with rope: dq and dk are turned back (by -theta) before they are stored
};

// Work list of (segment, tile) pairs, most work first (attn_sched.hip).
struct TileSchedule {
  int32_t* items;     // [4 * cap]: segment start, segment length, tile index, segment
  int32_t* hist;      // [n_bins]: tiles per work bin, then scatter cursors
  int32_t* toff;      // [n_seg + 1]: first tile of each segment (scan of tile counts)
  int32_t* n_items;   // [1]: tiles actually listed
  int64_t cap;
  int32_t n_bins;
};

size_t schedule_bytes(int64_t T, int32_t n_seg, int32_t max_seqlen, int tile, int unit);
TileSchedule schedule_carve(void* ws, int64_t T, int32_t n_seg, int32_t max_seqlen, int tile, int unit);
hipError_t launch_schedule(const int32_t* cu, int32_t n_seg, int32_t T, int tile, int unit, bool suffix,
                           const TileSchedule& s, hipStream_t stream);

size_t attn_fwd_workspace_bytes(int dtype, const AttnDims& d);
size_t attn_bwd_workspace_bytes(int dtype, const AttnDims& d);
hipError_t launch_attn_fwd_bf16(const AttnFwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnFwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_f32(const AttnBwdArgs& a, hipStream_t stream);

// Rotary embedding of q [T, hq, D] and k [T, hkv, D] in place (k may be null).
struct RopeArgs {
  int dtype;  // psc_dtype
  void* q;
  void* k;
  int64_t sq, sk, T;
  int32_t hq, hkv, d;
  int32_t inverse;
  const int32_t* pos;
  double inv_freq[64];  // base^(-2i/D), i < D/2
};
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);
// (cos, sin) table of positions [0, n_pos) for the attention kernels' turns.
hipError_t launch_rope_table(const RopeArgs& a, int32_t n_pos, float2* table, hipStream_t stream);

// unpack_data of packed rows [n_rows, packed_len] with the packer's flattened
// cu_seqlens (n_cu entries), row_seg_ptr and row_valid_len.
struct UnpackArgs {
  const int32_t *input_ids, *labels, *cu, *row_seg_ptr, *row_valid_len;
  int32_t *out_ids, *out_labels;
  int64_t n_rows, n_cu;
  int32_t packed_len, micro_bsz, seq_len;
};
hipError_t launch_unpack(const UnpackArgs& a, hipStream_t stream);
hipError_t launch_split(const int32_t* in, int64_t rows, int32_t length, int32_t tp, int32_t rank, int32_t* out,
                        hipStream_t stream);
hipError_t launch_row_max_seqlen(const int32_t* cu, int64_t n_cu, const int32_t* row_seg_ptr, int64_t n_rows,
                                 int32_t* out, hipStream_t stream);

// cu_seqlens check (validate.hip): flags[0] = OR of the kCu* bits that apply.
constexpr int32_t kCuBadStart = 1;       // c_0 != 0
constexpr int32_t kCuBadEnd = 2;         // c_n != T
constexpr int32_t kCuNotIncreasing = 4;  // some c_{i+1} <= c_i
hipError_t launch_check_cu(const int32_t* cu, int32_t n_seg, int32_t T, int32_t* flags, hipStream_t stream);

}  // namespace psc

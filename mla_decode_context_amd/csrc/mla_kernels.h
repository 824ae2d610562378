// Kernel parameter blocks and host-side launchers (internal to libmla).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeParams {
  const uint16_t* q_nope;  int64_t qn_st, qn_sh;   // element strides
  const uint16_t* q_pe;    int64_t qp_st, qp_sh;
  const uint16_t* kv;      int64_t kv_bs;          // block stride in elements
  int32_t P;                                        // page size (tokens per block)
  int32_t page_shift;                               // log2(P) if P is a power of two, else -1
  const int32_t* bt;       int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int32_t B, T, H, W, r;
  int32_t I;               // shard run length: token p lives on rank (p div I) mod W
  int32_t mode;            // kMaskCausal or kMaskContext (which keys a row sees)
  int32_t kv_fp8;          // cache rows hold FP8 E4M3 codes (576 bytes) instead of bf16
  float scale_log2;        // softmax scale * log2(e) (* the FP8 cache's scale): scores in base 2
  float out_scale;         // factor of the normalised output: the FP8 cache's scale, else 1
  int32_t chunk;           // keys per split (multiple of the 32-key step)
  int32_t hblocks;         // head blocks per query token
  int32_t max_splits;      // grid extent along splits
  uint16_t* out;           // bf16 [T,H,512] (when out_f is null)
  float* out_f;            // fp32 [T,H,512] partials instead of bf16, or null
  float* lse;              // fp32 [T,H]
  int32_t* row_keys;       // int32 [T]: each row's visible local keys, or null
  float* ws_o;             // fp32 [slots,H,512] split partials (normalised)
  float* ws_lse;           // fp32 [slots,H]
  int32_t* counters;       // int32 [T*hblocks] split tickets; zero between calls
  int4* row_desc;          // balanced schedule: per token {pieces, first slot, slot-0 offset, 0}
  int32_t* item_map;       // 128 heads: dispatch order, item of each grid position (-1: none); or null
  int2* item_info;         // with item_map: {request, the row's local keys} of each grid position
};

struct MergeParams {
  const uint16_t* outs;    // bf16 [W,T,H,512] (when outs_f is null)
  const float* outs_f;     // fp32 [W,T,H,512] partials instead, or null
  const float* lses;       // fp32 [W,T,H]
  const int32_t* valid;    // int32 [W,T] or null
  int32_t W, T, H;
  const uint16_t* wuv;     // bf16 [H,512,128] (merge + projection only)
  uint16_t* out;           // bf16 [T,H,512] or [T,H,128]
  float* out_lse;          // fp32 [T,H] or null
  int32_t hs;              // merge + projection: heads per output slice; head h goes to
                           // slice h / hs, laid out [H/hs][T][hs][128] (hs = H: [T][H][128])
};

// Combine of the projected slices one rank receives in the exchange: source s's
// rows [rows][128] at y + s*y_stride, their LSEs at lse + s*lse_stride.
struct SliceParams {
  const uint16_t* y;       int64_t y_stride;       // elements between sources
  const float* lse;        int64_t lse_stride;
  int32_t W, rows;         // sources; rows = T * heads of the slice
  uint16_t* out;           // bf16 [rows][128]
  float* out_lse;          // fp32 [rows] or null
};

// Heads handled by one decode workgroup: 16 * mtiles, mtiles in {1,2}.  With
// mtiles == 1 and workers > 0 the launch is `workers` workgroups that share
// the keys of all rows evenly (balanced schedule); otherwise the grid is
// (tokens * head blocks, max_splits) with fixed-size splits of p.chunk keys.
// The balanced launch is followed by a combine launch that merges the pieces
// of the rows it split.
hipError_t launch_decode(const DecodeParams& p, int mtiles, int max_splits, int workers, hipStream_t stream);
// 128 heads: one workgroup per (token, 64-head block, split), splits merged by
// a second launch.  With p.item_map set, a first one-workgroup launch orders the
// items longest first (the decode grid then runs them in that order).
hipError_t launch_decode_h128(const DecodeParams& p, hipStream_t stream);
hipError_t launch_local_seqlens(const int32_t* seq_lens, const int32_t* qsl, int B, int T, int W,
                                int r, int I, int mode, int32_t* row_seqlen, int32_t* shard_len, hipStream_t stream);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t stream);
hipError_t launch_lse_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_merge_v_up(const MergeParams& p, hipStream_t stream);
hipError_t launch_slice_combine(const SliceParams& p, hipStream_t stream);

}  // namespace mla

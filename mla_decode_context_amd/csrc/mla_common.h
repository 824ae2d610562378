// Device-side helpers shared by the gfx950 kernels of the MLA DCP decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kLatent = 512;   // c_kv / q_nope / output width (kv_lora_rank)
constexpr int kRope = 64;      // k_pe / q_pe width (qk_rope_head_dim)
constexpr int kRow = 576;      // one cache row, in bf16 elements
constexpr int kVHead = 128;    // width after the W_UV up-projection

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // One packed round-to-nearest-even conversion of both halves.
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Where query token t sits and how many keys it sees on DCP rank r of W.
//
// Requests own contiguous token ranges [qsl[b], qsl[b+1]); S_b = seq_lens[b] is
// the request's global token count including its Q_b query tokens, which are
// its last Q_b tokens, so row i is at global position p = S_b - Q_b + i and
// sees the global keys 0..p.  Rank r stores the keys r, r+W, ..., so the row
// sees the first ceil((p + 1 - r) / W) of the rank's local keys (none when
// p < r); the rank stores ceil((S_b - r) / W) of the request's tokens.
struct RowInfo {
  int b;        // request
  int L;        // visible local keys of this row on rank r
};

// Mask modes of a decode call.  kMaskCausal: row i of a request (global
// position p = S - Q + i) sees the keys 0..p (per rank, the interleaved DCP
// mask).  kMaskContext: every row of the request sees the keys 0..S-Q-1, its
// tokens before the query tokens, without a causal mask (the context stage of
// the two-stage split of a decode with more than one query row).
constexpr int kMaskCausal = 0;
constexpr int kMaskContext = 1;

__device__ __forceinline__ int ceil_div_pos(int n, int W) { return n > 0 ? (n + W - 1) / W : 0; }

// Shard layout: runs of I consecutive tokens of a request are dealt to the W
// ranks in turn, so global token p lives on rank (p div I) mod W -- I = 1 is the
// interleaved layout (token p on rank p mod W), I = page size gives each rank
// whole pages.  Of the positions 0..n-1 rank r holds
//   (n div WI) * I + min(max(n mod WI - rI, 0), I),
// and they are the first ones of its local order (ascending position).
__device__ __forceinline__ int shard_count(int n, int W, int r, int I) {
  if (n <= 0) return 0;
  if (I == 1) return ceil_div_pos(n - r, W);
  const int span = W * I;
  const int rounds = n / span;
  return rounds * I + min(max(n - rounds * span - r * I, 0), I);
}

// Global position of rank r's local token j (the inverse of the layout above).
__device__ __forceinline__ int shard_position(int j, int W, int r, int I) {
  if (I == 1) return j * W + r;
  const int run = j / I;
  return (run * W + r) * I + (j - run * I);
}

// Local keys that row i of a request (S tokens, Q query rows) sees on rank r:
// a prefix of the rank's local order under either mask mode.
__device__ __forceinline__ int row_key_count(int S, int Q, int i, int W, int r, int I, int mode) {
  return shard_count(mode == kMaskContext ? S - Q : S - Q + i + 1, W, r, I);
}

__device__ __forceinline__ RowInfo locate_row(const int32_t* __restrict__ qsl,
                                              const int32_t* __restrict__ seq_lens,
                                              int B, int t, int W, int r, int I, int mode) {
  // last b with qsl[b] <= t; it has qsl[b+1] > t because t < qsl[B]
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int q0 = qsl[lo];
  const int q = qsl[lo + 1] - q0;
  RowInfo ri;
  ri.b = lo;
  ri.L = row_key_count(seq_lens[lo], q, t - q0, W, r, I, mode);
  return ri;
}

}  // namespace mla

// C ABI of libmla: argument validation, launch planning and kernel launches.
// The call contracts are documented in include/mla.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "mla.h"
#include "mla_kernels.h"

// Scratch of mla_decode_partial_noalloc: one copy in every GPU's memory,
// held until the process ends.  In host code `scratch` is only a handle for
// hipGetSymbolAddress; the address on each device is looked up once and kept
// in g_scratch (the kernels take it as an argument).
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
int g_device_state[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other

mla_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  int st = __atomic_load_n(&g_device_state[dev], __ATOMIC_ACQUIRE);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    __atomic_store_n(&g_device_state[dev], st, __ATOMIC_RELEASE);
  }
  return st == 1 ? MLA_OK : MLA_ERR_UNSUPPORTED;
}

// Device address of `scratch` on each device (looked up on the first
// mla_decode_partial_noalloc call made with that device current).
struct ScratchSlot {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];

mla_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s] {
    s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch));
    if (s.err != hipSuccess) s.ptr = nullptr;
  });
  if (s.err != hipSuccess || s.ptr == nullptr) return MLA_ERR_HIP;
  *out = s.ptr;
  return MLA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

constexpr int kStep = 32;          // keys per inner step of the decode kernel
constexpr int kTargetGroups = 512;   // busy workgroups wanted per launch (2 per CU)
constexpr int kMinChunk = 1024;    // auto splits never go below this many keys
constexpr int kMaxGridY = 65535;
// Balanced schedule of the 16-head kernel: one workgroup per CU of the
// 256-CU part (the kernel's LDS allows one per CU).
constexpr int kWorkers = 256;
// 128-head kernel (64 or 128 heads, one workgroup per 64-head block): one
// workgroup per CU; automatic splits aim for 2 * kH128Groups workgroups (rows x
// head blocks x splits) and never cut a row below kH128MinChunk keys.
constexpr int kH128Groups = 256;
constexpr int kH128MinChunk = 512;
constexpr int kH128Stage = 32;

// Launch plan: heads per workgroup and how keys are split.  Depends only on
// host integers so that the workspace size can be computed in advance.
struct Plan {
  bool h128;        // the 128-head kernel (one workgroup per token and split)
  int mtiles;       // 16-head tiles per workgroup (1 or 2)
  int hblocks;      // workgroups per token along heads
  int chunk;        // keys per split (fixed-split grid)
  int max_splits;   // grid extent along splits (fixed-split grid)
  int workers;      // > 0: balanced schedule over this many workgroups
  bool ordered;     // 64 or 128 heads: longest-first dispatch order in the workspace
};

// The 128-head kernel's dispatch order sorts (split, request) units in one
// workgroup's LDS; more units than this run in token order.
constexpr int64_t kH128MaxOrderUnits = 8192;

// Of the positions 0..n-1, the tokens that runs of I dealt to W ranks in turn
// put on rank r (the device's shard_count, on the host).
int64_t host_shard_count(int64_t n, int64_t W, int64_t r, int64_t I) {
  if (n <= 0) return 0;
  const int64_t rounds = n / (W * I);
  const int64_t m = n - rounds * W * I - r * I;
  return rounds * I + (m < 0 ? 0 : m > I ? I : m);
}

// A shard layout the kernels can index: W ranks, runs of I tokens, W * I in int.
bool layout_ok(int32_t W, int32_t I) { return W >= 1 && I >= 1 && (int64_t)W * I <= (int64_t(1) << 30); }

Plan make_plan(int B, int T, int H, int max_seq_len, int W, int I, int num_splits, bool split_ok) {
  Plan p;
  const int ht = (H + 15) / 16;
  p.mtiles = ht >= 2 ? 2 : 1;
  p.hblocks = (int)ceil_div(ht, p.mtiles);
  p.workers = 0;
  p.h128 = H % 64 == 0;           // 64 or 128 heads: the 128-head kernel, one workgroup per 64-head block
  if (p.h128) p.hblocks = H / 64;
  // A row's visible local keys never exceed what rank 0 (the first run of every
  // round) holds of max_seq_len tokens: ceil(max_seq_len / W) when I = 1.
  const int64_t lmax = host_shard_count(max_seq_len, W, 0, I);
  const int64_t lr = round_up(lmax > 0 ? lmax : 1, kStep);
  int64_t chunk = lr;
  if (p.h128) {
    // A split's partial is 128 KiB per 64-head block (64 heads x 512 fp32):
    // split only when there are too few rows to fill the CUs, or when asked
    // to.  Splits are multiples of the kernel's 32-key stage.
    if (split_ok && lmax > 0 && num_splits != 1) {
      if (num_splits > 1) {
        chunk = round_up(ceil_div(lmax, num_splits), kH128Stage);
      } else {
        const int64_t want = ceil_div(2 * kH128Groups, (T > 0 ? T : 1) * (int64_t)p.hblocks);
        if (want > 1) chunk = round_up(ceil_div(lmax, want), kH128Stage);
        if (chunk < kH128MinChunk) chunk = kH128MinChunk;
      }
      if (chunk >= lmax) chunk = lr;
    }
  } else if (split_ok && num_splits == 0 && p.mtiles == 1) {
    p.workers = kWorkers;
  } else if (split_ok && num_splits != 1 && lmax > 0) {
    if (num_splits > 1) {
      chunk = round_up(ceil_div(lmax, num_splits), kStep);
    } else {
      // Rows are on average about half as long as the bound; aim for
      // kTargetGroups busy workgroups.
      const int64_t base = (int64_t)T * p.hblocks;
      const int64_t want = ceil_div(2 * kTargetGroups, base > 0 ? base : 1);
      if (want > 1) chunk = round_up(ceil_div(lmax, want), kStep);
      if (chunk < kMinChunk) chunk = kMinChunk;
    }
    if (chunk > lr) chunk = lr;
    if (ceil_div(lr, chunk) > kMaxGridY) chunk = round_up(ceil_div(lr, kMaxGridY), kStep);
  }
  p.chunk = (int)chunk;
  p.max_splits = (int)ceil_div(lr, chunk);
  p.ordered = p.h128 && split_ok && (int64_t)B * p.max_splits <= kH128MaxOrderUnits;
  return p;
}

// Workspace layout (offsets from the 256-byte aligned base):
//   int32 item_map[T * hblocks * max_splits]  64 or 128 heads only: dispatch order
//   int2  item_info[T * hblocks * max_splits] 64 or 128 heads only: {request, keys} per position
//   int32 counters[T * hblocks]          split tickets, zero between calls
//   int4  row_desc[T]                    balanced schedule only: pieces per row
//   fp32  lse[slots][H]                  split LSEs
//   fp32  o[slots][H][512]               normalised split partials
// with slots = max_splits * T (fixed splits; slot split*T + t) or 2 * workers
// (balanced schedule; two per workgroup).  The split regions exist only when
// the plan splits.
bool splits_ws(const Plan& p) { return p.workers > 0 || p.max_splits > 1; }
// Plans whose split rows merge through ticketed last-arriver workgroups
// (fixed splits of the 16-head and generic kernels).
bool uses_tickets(const Plan& p) { return !p.h128 && p.workers == 0 && p.max_splits > 1; }
bool uses_workspace(const Plan& p) { return splits_ws(p) || p.ordered; }
int64_t slots_of(const Plan& p, int T) { return p.workers > 0 ? 2 * (int64_t)p.workers : (int64_t)p.max_splits * T; }
size_t map_bytes(const Plan& p, int T) {
  return p.ordered ? (size_t)round_up((int64_t)T * p.hblocks * p.max_splits * 4, 256) : 0;
}
size_t info_bytes(const Plan& p, int T) {
  return p.ordered ? (size_t)round_up((int64_t)T * p.hblocks * p.max_splits * 8, 256) : 0;
}
size_t counters_bytes(const Plan& p, int T) { return (size_t)round_up((int64_t)T * p.hblocks * 4, 256); }
size_t desc_bytes(const Plan& p, int T) { return p.workers > 0 ? (size_t)round_up((int64_t)T * 16, 256) : 0; }
size_t lse_bytes(const Plan& p, int T, int H) { return (size_t)round_up(slots_of(p, T) * H * 4, 256); }

size_t workspace_bytes_for(const Plan& p, int T, int H) {
  if (!uses_workspace(p)) return 0;
  size_t n = map_bytes(p, T) + info_bytes(p, T) + 256;
  if (splits_ws(p)) {
    const size_t rows = (size_t)slots_of(p, T) * H;
    n += counters_bytes(p, T) + desc_bytes(p, T) + lse_bytes(p, T, H) + rows * MLA_D_LATENT * sizeof(float);
  }
  return n;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool dtype_ok(int32_t d) { return d == MLA_DTYPE_BF16 || d == MLA_DTYPE_F32; }
bool mask_ok(int32_t m) { return m == MLA_MASK_CAUSAL || m == MLA_MASK_CONTEXT; }

mla_status fail(char* reason, size_t len, const char* fmt, ...) {
  if (reason && len > 0) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(reason, len, fmt, ap);
    va_end(ap);
  }
  return MLA_ERR_SHAPE;
}

bool debug_mode() {
  const char* v = getenv("MLA_DEBUG");
  return v && v[0] == '1' && v[1] == 0;
}

// Blocks of the allocation that holds kv_cache, from kv_cache on (a block k is
// usable when its page_size rows end inside the allocation); -1 if unknown.
int64_t blocks_in_allocation(const void* kv_cache, int64_t kv_block_stride, int32_t page_size, int elem_bytes) {
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)kv_cache) != hipSuccess || !base) {
    (void)hipGetLastError();
    return -1;
  }
  const int64_t avail = (int64_t)((uintptr_t)base + size - (uintptr_t)kv_cache);
  const int64_t block = (int64_t)page_size * MLA_D_ROW * elem_bytes;
  if (avail < block) return 0;
  return (avail - block) / (kv_block_stride * elem_bytes) + 1;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: a size, stride, rank or alignment is out of range";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: the current device is not gfx950";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small for the split plan";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case MLA_ERR_CAPTURE: return "MLA_ERR_CAPTURE: MLA_DEBUG checks cannot run on a capturing stream";
    default: return "unknown mla_status";
  }
}

mla_status mla_check_decode_metadata(const int32_t* seq_lens, const int32_t* query_start_loc,
                                     const int32_t* block_table, int32_t bt_stride, int32_t B, int32_t T,
                                     int32_t max_query_len, int32_t max_seq_len, int32_t page_size,
                                     int32_t cp_world, int32_t cp_rank, int32_t cp_interleave,
                                     int32_t mask_mode, int64_t num_blocks, char* reason, size_t reason_len) {
  if (reason && reason_len) reason[0] = 0;
  if (B < 0 || T < 0 || page_size < 1 || !layout_ok(cp_world, cp_interleave) || cp_rank < 0 ||
      cp_rank >= cp_world || bt_stride < 1 || !mask_ok(mask_mode))
    return fail(reason, reason_len, "invalid sizes");
  if (B == 0) return T == 0 ? MLA_OK : fail(reason, reason_len, "T = %d tokens without requests", T);
  if (!seq_lens || !query_start_loc || !block_table) return MLA_ERR_NULL;
  if (query_start_loc[0] != 0)
    return fail(reason, reason_len, "query_start_loc[0] = %d, not 0", query_start_loc[0]);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t q = query_start_loc[b + 1] - query_start_loc[b];
    if (q < 0)
      return fail(reason, reason_len, "query_start_loc decreases at request %d (%d -> %d)", b,
                  query_start_loc[b], query_start_loc[b + 1]);
    if (q > max_query_len)
      return fail(reason, reason_len, "request %d has %d query rows > max_query_len %d", b, q, max_query_len);
    const int32_t S = seq_lens[b];
    if (S < q) return fail(reason, reason_len, "request %d: seq_len %d < its %d query rows", b, S, q);
    if (S > max_seq_len)
      return fail(reason, reason_len, "request %d: seq_len %d > max_seq_len %d", b, S, max_seq_len);
    const int64_t lc = host_shard_count(mask_mode == MLA_MASK_CONTEXT ? S - q : S, cp_world, cp_rank, cp_interleave);
    const int64_t nb = ceil_div(lc, page_size);
    if (nb > bt_stride)
      return fail(reason, reason_len, "request %d needs %lld blocks on rank %d, the block table row has %d", b,
                  (long long)nb, cp_rank, bt_stride);
    for (int64_t i = 0; i < nb; ++i) {
      const int32_t id = block_table[(int64_t)b * bt_stride + i];
      if (id < 0 || (num_blocks >= 0 && id >= num_blocks))
        return fail(reason, reason_len, "request %d: block_table entry %lld = %d outside [0, %lld)", b,
                    (long long)i, id, (long long)(num_blocks >= 0 ? num_blocks : (int64_t)1 << 31));
    }
  }
  if (query_start_loc[B] != T)
    return fail(reason, reason_len, "query_start_loc[B] = %d, not T = %d", query_start_loc[B], T);
  return MLA_OK;
}

size_t mla_decode_workspace_size(int32_t B, int32_t T, int32_t H, int32_t max_query_len,
                                 int32_t max_seq_len, int32_t cp_world, int32_t cp_interleave,
                                 int32_t num_splits) {
  if (B < 0 || T < 0 || H < 1 || H > MLA_MAX_HEADS || max_query_len < 0 || max_seq_len < 0 ||
      !layout_ok(cp_world, cp_interleave) || num_splits < 0)
    return (size_t)-1;
  if (B == 0 || T == 0) return 0;
  const Plan p = make_plan(B, T, H, max_seq_len, cp_world, cp_interleave, num_splits, true);
  return workspace_bytes_for(p, T, H);
}

}  // extern "C"

// mla_decode_partial and mla_decode_partial_noalloc: the same checks, plan
// and kernels; `noalloc` takes the workspace from this device's scratch array
// (never MLA_DEBUG, whose host copies would allocate).
static mla_status decode_impl(
    const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
    const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
    const void* kv_cache, int32_t kv_dtype, float kv_scale, int64_t kv_block_stride, int32_t page_size,
    const int32_t* block_table, int32_t bt_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    int32_t B, int32_t T, int32_t H, int32_t max_query_len, int32_t max_seq_len,
    int32_t cp_world, int32_t cp_rank, int32_t cp_interleave, int32_t mask_mode, float scale,
    int32_t num_splits,
    void* out, int32_t out_dtype, float* lse, int32_t* row_keys,
    void* workspace, size_t workspace_bytes, void* hip_stream, bool noalloc) {
  if (B < 0 || T < 0 || H < 1 || H > MLA_MAX_HEADS || page_size < 1 || !layout_ok(cp_world, cp_interleave) ||
      cp_rank < 0 || cp_rank >= cp_world || max_query_len < 0 || max_seq_len < 0 ||
      num_splits < 0 || !isfinite(scale) || !(scale > 0.f) || !dtype_ok(out_dtype) || !mask_ok(mask_mode))
    return MLA_ERR_SHAPE;
  if (B == 0 && T > 0) return MLA_ERR_SHAPE;   // tokens without requests
  if (B == 0 || T == 0) return MLA_OK;
  if (!q_nope || !q_pe || !kv_cache || !block_table || !seq_lens || !query_start_loc || !out || !lse)
    return MLA_ERR_NULL;
  // Vector loads need 16-byte rows of q_nope / cache and 8-byte rows of q_pe.
  if (qn_stride_h < MLA_D_LATENT || qn_stride_t < (int64_t)H * qn_stride_h || qn_stride_h % 8 ||
      qn_stride_t % 8 || !aligned(q_nope, 16))
    return MLA_ERR_SHAPE;
  if (qp_stride_h < MLA_D_ROPE || qp_stride_t < (int64_t)(H - 1) * qp_stride_h + MLA_D_ROPE ||
      qp_stride_h % 4 || qp_stride_t % 4 || !aligned(q_pe, 8))
    return MLA_ERR_SHAPE;
  const bool fp8 = kv_dtype == MLA_DTYPE_FP8_E4M3;
  if (kv_dtype != MLA_DTYPE_BF16 && !fp8) return MLA_ERR_SHAPE;
  if (fp8 && (!isfinite(kv_scale) || !(kv_scale > 0.f))) return MLA_ERR_SHAPE;
  if (kv_block_stride < (int64_t)page_size * MLA_D_ROW || kv_block_stride % (fp8 ? 16 : 8) || !aligned(kv_cache, 16))
    return MLA_ERR_SHAPE;
  if (fp8 && H > 16) return MLA_ERR_UNSUPPORTED;
  if (bt_stride < 1 || !aligned(out, 16)) return MLA_ERR_SHAPE;
  mla_status st = check_device();
  if (st != MLA_OK) return st;
  if (!noalloc && debug_mode()) {
    // Host copies of the metadata, one wait, the contract checked before
    // anything is enqueued.  Not valid inside capture.
    hipStream_t s = (hipStream_t)hip_stream;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return MLA_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return MLA_ERR_CAPTURE;
    std::vector<int32_t> hs(B), hq(B + 1), hb((size_t)B * bt_stride);
    if (hipMemcpyAsync(hs.data(), seq_lens, hs.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(hq.data(), query_start_loc, hq.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(hb.data(), block_table, hb.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return MLA_ERR_HIP;
    char why[256];
    const mla_status cst = mla_check_decode_metadata(
        hs.data(), hq.data(), hb.data(), bt_stride, B, T, max_query_len, max_seq_len, page_size, cp_world, cp_rank,
        cp_interleave, mask_mode, blocks_in_allocation(kv_cache, kv_block_stride, page_size, fp8 ? 1 : 2), why,
        sizeof(why));
    if (cst != MLA_OK) {
      fprintf(stderr, "mla_decode_partial (MLA_DEBUG): %s\n", why);
      return cst;
    }
  }

  const Plan plan = make_plan(B, T, H, max_seq_len, cp_world, cp_interleave, num_splits,
                              noalloc || workspace != nullptr);
  const size_t need = workspace_bytes_for(plan, T, H);
  if (noalloc) {
    if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
    if (need > 0) {
      st = scratch_address(&workspace);
      if (st != MLA_OK) return st;
      workspace_bytes = MLA_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (need > 0 && workspace_bytes < need) return MLA_ERR_WORKSPACE;

  mla::DecodeParams p;
  p.q_nope = (const uint16_t*)q_nope; p.qn_st = qn_stride_t; p.qn_sh = qn_stride_h;
  p.q_pe = (const uint16_t*)q_pe; p.qp_st = qp_stride_t; p.qp_sh = qp_stride_h;
  p.kv = (const uint16_t*)kv_cache; p.kv_bs = kv_block_stride; p.P = page_size;
  p.page_shift = (page_size & (page_size - 1)) == 0 ? __builtin_ctz((unsigned)page_size) : -1;
  p.bt = block_table; p.bt_stride = bt_stride;
  p.seq_lens = seq_lens; p.qsl = query_start_loc;
  p.B = B; p.T = T; p.H = H; p.W = cp_world; p.r = cp_rank; p.I = cp_interleave; p.mode = mask_mode;
  p.kv_fp8 = fp8 ? 1 : 0;
  p.scale_log2 = (float)((double)scale * (fp8 ? (double)kv_scale : 1.0) * 1.4426950408889634074);
  p.out_scale = fp8 ? kv_scale : 1.f;
  p.chunk = plan.chunk; p.hblocks = plan.hblocks; p.max_splits = plan.max_splits;
  p.out = out_dtype == MLA_DTYPE_BF16 ? (uint16_t*)out : nullptr;
  p.out_f = out_dtype == MLA_DTYPE_F32 ? (float*)out : nullptr;
  p.lse = lse;
  p.row_keys = row_keys;
  p.ws_o = nullptr; p.ws_lse = nullptr; p.counters = nullptr; p.row_desc = nullptr; p.item_map = nullptr;
  p.item_info = nullptr;
  char* ws_base = (char*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  if (plan.ordered) {
    p.item_map = (int32_t*)ws_base;
    p.item_info = (int2*)(ws_base + map_bytes(plan, T));
  }
  if (splits_ws(plan)) {
    char* base = ws_base + map_bytes(plan, T) + info_bytes(plan, T);
    const size_t c_end = counters_bytes(plan, T);
    const size_t d_end = c_end + desc_bytes(plan, T);
    p.counters = (int32_t*)base;
    p.row_desc = plan.workers > 0 ? (int4*)(base + c_end) : nullptr;
    p.ws_lse = (float*)(base + d_end);
    p.ws_o = (float*)(base + d_end + lse_bytes(plan, T, H));
  }
  if (noalloc && uses_tickets(plan)) {
    // The split tickets must start at zero; a caller-owned workspace is
    // zero-filled once by its owner, the scratch array is cleared here (a
    // kernel, so the call stays capturable).
    const hipError_t ez = mla::launch_zero_i32(p.counters, (int)(counters_bytes(plan, T) / 4), (hipStream_t)hip_stream);
    if (ez != hipSuccess) return MLA_ERR_HIP;
  }
  hipError_t e = plan.h128 ? mla::launch_decode_h128(p, (hipStream_t)hip_stream)
                           : mla::launch_decode(p, plan.mtiles, plan.max_splits, plan.workers, (hipStream_t)hip_stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" {

mla_status mla_decode_partial(
    const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
    const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
    const void* kv_cache, int32_t kv_dtype, float kv_scale, int64_t kv_block_stride, int32_t page_size,
    const int32_t* block_table, int32_t bt_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    int32_t B, int32_t T, int32_t H, int32_t max_query_len, int32_t max_seq_len,
    int32_t cp_world, int32_t cp_rank, int32_t cp_interleave, int32_t mask_mode, float scale,
    int32_t num_splits,
    void* out, int32_t out_dtype, float* lse, int32_t* row_keys,
    void* workspace, size_t workspace_bytes, void* hip_stream) {
  return decode_impl(q_nope, qn_stride_t, qn_stride_h, q_pe, qp_stride_t, qp_stride_h, kv_cache, kv_dtype, kv_scale,
                     kv_block_stride,
                     page_size, block_table, bt_stride, seq_lens, query_start_loc, B, T, H, max_query_len,
                     max_seq_len, cp_world, cp_rank, cp_interleave, mask_mode, scale, num_splits, out, out_dtype, lse, row_keys,
                     workspace, workspace_bytes, hip_stream, false);
}

mla_status mla_decode_partial_noalloc(
    const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
    const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
    const void* kv_cache, int32_t kv_dtype, float kv_scale, int64_t kv_block_stride, int32_t page_size,
    const int32_t* block_table, int32_t bt_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    int32_t B, int32_t T, int32_t H, int32_t max_query_len, int32_t max_seq_len,
    int32_t cp_world, int32_t cp_rank, int32_t cp_interleave, int32_t mask_mode, float scale,
    int32_t num_splits,
    void* out, int32_t out_dtype, float* lse, int32_t* row_keys, void* hip_stream) {
  return decode_impl(q_nope, qn_stride_t, qn_stride_h, q_pe, qp_stride_t, qp_stride_h, kv_cache, kv_dtype, kv_scale,
                     kv_block_stride,
                     page_size, block_table, bt_stride, seq_lens, query_start_loc, B, T, H, max_query_len,
                     max_seq_len, cp_world, cp_rank, cp_interleave, mask_mode, scale, num_splits, out, out_dtype, lse, row_keys,
                     nullptr, 0, hip_stream, true);
}

static mla_status merge_common(const void* outs, int32_t outs_dtype, const float* lses, const int32_t* valid,
                               int32_t W, int32_t T, int32_t H, const void* W_UV, bool proj, void* out,
                               float* out_lse, void* hip_stream) {
  if (W < 1 || T < 0 || H < 1 || H > MLA_MAX_HEADS || !dtype_ok(outs_dtype)) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!outs || !lses || !out || (proj && !W_UV)) return MLA_ERR_NULL;
  if (!aligned(outs, 16) || !aligned(out, 16) || (proj && !aligned(W_UV, 16))) return MLA_ERR_SHAPE;
  mla_status st = check_device();
  if (st != MLA_OK) return st;
  mla::MergeParams p;
  p.outs = outs_dtype == MLA_DTYPE_BF16 ? (const uint16_t*)outs : nullptr;
  p.outs_f = outs_dtype == MLA_DTYPE_F32 ? (const float*)outs : nullptr;
  p.lses = lses; p.valid = valid;
  p.W = W; p.T = T; p.H = H;
  p.wuv = (const uint16_t*)W_UV; p.out = (uint16_t*)out; p.out_lse = out_lse; p.hs = H;
  hipError_t e = proj ? mla::launch_merge_v_up(p, (hipStream_t)hip_stream)
                      : mla::launch_lse_merge(p, (hipStream_t)hip_stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_lse_merge(const void* outs, int32_t outs_dtype, const float* lses, const int32_t* valid,
                         int32_t W, int32_t T, int32_t H,
                         void* out, float* out_lse, void* hip_stream) {
  return merge_common(outs, outs_dtype, lses, valid, W, T, H, nullptr, false, out, out_lse, hip_stream);
}

mla_status mla_merge_v_up_proj(const void* outs, int32_t outs_dtype, const float* lses, const int32_t* valid,
                               int32_t W, int32_t T, int32_t H, const void* W_UV,
                               void* out, float* out_lse, void* hip_stream) {
  return merge_common(outs, outs_dtype, lses, valid, W, T, H, W_UV, true, out, out_lse, hip_stream);
}

mla_status mla_dcp_a2a_pack(const void* out_r, int32_t out_dtype, const float* lse_r, const int32_t* valid_r,
                            int32_t T, int32_t H, int32_t cp_world, const void* W_UV,
                            void* send_y, float* send_lse, void* hip_stream) {
  if (T < 0 || H < 1 || H > MLA_MAX_HEADS || cp_world < 1 || H % cp_world != 0 || !dtype_ok(out_dtype))
    return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!out_r || !lse_r || !W_UV || !send_y || !send_lse) return MLA_ERR_NULL;
  if (!aligned(out_r, 16) || !aligned(send_y, 16) || !aligned(W_UV, 16)) return MLA_ERR_SHAPE;
  mla_status st = check_device();
  if (st != MLA_OK) return st;
  // The fused merge + projection over one partial (its merge is the identity),
  // writing head h into destination slice h / (H / cp_world).
  mla::MergeParams p;
  p.outs = out_dtype == MLA_DTYPE_BF16 ? (const uint16_t*)out_r : nullptr;
  p.outs_f = out_dtype == MLA_DTYPE_F32 ? (const float*)out_r : nullptr;
  p.lses = lse_r; p.valid = valid_r;
  p.W = 1; p.T = T; p.H = H;
  p.wuv = (const uint16_t*)W_UV; p.out = (uint16_t*)send_y; p.out_lse = send_lse; p.hs = H / cp_world;
  return mla::launch_merge_v_up(p, (hipStream_t)hip_stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_dcp_a2a_combine(const void* recv_y, int64_t recv_y_stride, const float* recv_lse,
                               int64_t recv_lse_stride, int32_t cp_world, int32_t T, int32_t Hs,
                               void* out, float* out_lse, void* hip_stream) {
  if (cp_world < 1 || T < 0 || Hs < 1 || Hs > MLA_MAX_HEADS) return MLA_ERR_SHAPE;
  const int64_t rows = (int64_t)T * Hs;
  if (rows == 0) return MLA_OK;
  if (!recv_y || !recv_lse || !out) return MLA_ERR_NULL;
  if (cp_world > 1 && (recv_y_stride < rows * MLA_D_V || recv_lse_stride < rows)) return MLA_ERR_SHAPE;
  if (recv_y_stride % 8 != 0 || !aligned(recv_y, 16) || !aligned(out, 16)) return MLA_ERR_SHAPE;
  mla_status st = check_device();
  if (st != MLA_OK) return st;
  mla::SliceParams p;
  p.y = (const uint16_t*)recv_y; p.y_stride = recv_y_stride;
  p.lse = recv_lse; p.lse_stride = recv_lse_stride;
  p.W = cp_world; p.rows = (int32_t)rows;
  p.out = (uint16_t*)out; p.out_lse = out_lse;
  return mla::launch_slice_combine(p, (hipStream_t)hip_stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_dcp_local_seqlens(const int32_t* seq_lens, const int32_t* query_start_loc,
                                 int32_t B, int32_t T, int32_t cp_world, int32_t cp_rank,
                                 int32_t cp_interleave, int32_t mask_mode, int32_t* row_seqlen,
                                 int32_t* shard_len, void* hip_stream) {
  if (B < 0 || T < 0 || !layout_ok(cp_world, cp_interleave) || cp_rank < 0 || cp_rank >= cp_world ||
      !mask_ok(mask_mode))
    return MLA_ERR_SHAPE;
  if (B == 0 && T > 0) return MLA_ERR_SHAPE;
  if (B == 0 && T == 0) return MLA_OK;
  if (!seq_lens || !query_start_loc) return MLA_ERR_NULL;
  mla_status st = check_device();
  if (st != MLA_OK) return st;
  hipError_t e = mla::launch_local_seqlens(seq_lens, query_start_loc, B, T, cp_world, cp_rank,
                                           cp_interleave, mask_mode, row_seqlen, shard_len, (hipStream_t)hip_stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

// Exact LSE-weighted merge of per-rank DCP partials, alone and fused with the
// per-head W_UV up-projection, for gfx950 (CDNA4).
//
// What is computed follows PR #48196 ("DCP sparse MLA output-merge
// optimizations"): the merge weights each rank's partial by exp(lse_r - LSE)
// with LSE = ln sum_r exp(lse_r), ranks whose per-row valid count is zero take
// no part (their buffers are not read), and the W_UV projection is linear, so
// projecting the merged latent row equals merging the projected partials.
//
// Both kernels stream the partials once from HBM (the merge is bandwidth-bound:
// about W*1 KiB read per (token, head) against 1 KiB or 256 B written).
#include "mla_common.h"
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

// Workgroup = (8 heads, a contiguous range of tokens), 256 threads; thread
// (head 8*blockIdx.x + tid / 32, dims 16*(tid % 32) .. +16).  The workgroup
// walks its tokens in items of (token, R ranks): every rank's LSE and partial
// of the item are loaded together and combined online (running max, rescaled
// sum, ranks in order).  Three register buffers rotate so that two items'
// loads are in flight while one is combined.  Whether rank w takes part in
// row t is the same for the whole workgroup, so valid[w, t] comes through
// scalar loads one item earlier still.  Every load and store is a buffer
// operation issued whether or not its lane has work: a disabled lane carries
// an offset past the buffer's range, which reads zero (or writes nothing)
// without touching memory, so the compiler's waits for the loads stay exact.
// R = 4 when W <= 8 (fewer registers, more workgroups per CU; ranks 5..8 are a
// second item of the same token), else 8; with fp32 partials (kF32: twice the
// bytes per rank) half as many, so an item holds the same bytes.
constexpr int kMergeHeads = 8;
constexpr int kBufFlags = 0x00020000;              // buffer resource word 3 (raw 32-bit data)
constexpr uint32_t kOffNone = 0x40000000u;         // past every buffer range used here

// 16 partial values of one rank as loaded (bf16: two 16-byte words; fp32:
// four), as four fp32 vectors.
template <bool kF32>
__device__ __forceinline__ void unpack16(const u32x4* x, f32x4 (&v)[4]) {
  if constexpr (kF32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_bit_cast(f32x4, x[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      v[2 * k] = f32x4{bf16_lo(x[k][0]), bf16_hi(x[k][0]), bf16_lo(x[k][1]), bf16_hi(x[k][1])};
      v[2 * k + 1] = f32x4{bf16_lo(x[k][2]), bf16_hi(x[k][2]), bf16_lo(x[k][3]), bf16_hi(x[k][3])};
    }
  }
}

// acc = acc * c_old + x * c_new over the 16 values.
template <bool kF32>
__device__ __forceinline__ void axpy16(f32x4 (&acc)[4], float c_old, const u32x4* x, float c_new) {
  f32x4 v[4];
  unpack16<kF32>(x, v);
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = acc[k] * c_old + v[k] * c_new;
}

template <int R, bool kValid, bool kF32>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeParams a) {
  constexpr int kWords = kF32 ? 4 : 2;               // 16-byte loads per 16 values
  constexpr int kElem = kF32 ? 4 : 2;                // bytes per partial value
  const uint8_t* outs = kF32 ? (const uint8_t*)a.outs_f : (const uint8_t*)a.outs;
  const int hl = threadIdx.x >> 5;
  const int h0 = kMergeHeads * (int)blockIdx.x;
  const bool hok = h0 + hl < a.H;
  const int d0 = 16 * (threadIdx.x & 31);
  const int per = (a.T + (int)gridDim.y - 1) / (int)gridDim.y;
  const int t_begin = (int)blockIdx.y * per;
  const int t_end = min(a.T, t_begin + per);
  if (t_begin >= t_end) return;
  const size_t plane = (size_t)a.T * a.H;
  const int ngroups = (a.W + R - 1) / R;
  const int nitems = (t_end - t_begin) * ngroups;
  struct Pend {
    u32x4 x[R][kWords];
    float l[R];
    int part;          // bit u: rank w0 + u was read
  };
  auto item_t = [&](int i) { return min(t_begin + i / ngroups, a.T - 1); };
  auto load_valid = [&](int i, int (&vv)[R]) {
    const int t = item_t(i), w0 = R * (i % ngroups);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int w = min(w0 + u, a.W - 1);
      int c = 1;
      if (kValid) c = ((const __attribute__((address_space(4))) int32_t*)a.valid)[(size_t)w * a.T + t] > 0 ? 1 : 0;
      vv[u] = c & ((i < nitems && w0 + u < a.W && hok) ? 1 : 0);
    }
  };
  auto load_data = [&](int i, const int (&vv)[R], Pend& p) {
    const int t = item_t(i), w0 = R * (i % ngroups);
    p.part = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const size_t row0 = min(w0 + u, a.W - 1) * plane + (size_t)t * a.H + h0;   // the item's first head
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(outs + row0 * kLatent * kElem), (short)0, kMergeHeads * kLatent * kElem, kBufFlags);
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.lses + row0), (short)0, kMergeHeads * 4, kBufFlags);
      const uint32_t oo = vv[u] ? (uint32_t)(hl * kLatent * kElem + kElem * d0) : kOffNone;
      const uint32_t ol = vv[u] ? (uint32_t)(hl * 4) : kOffNone;
      p.l[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, ol, 0, 0));
#pragma unroll
      for (int k = 0; k < kWords; ++k) p.x[u][k] = __builtin_amdgcn_raw_buffer_load_b128(ro, oo + 16 * k, 0, 0);
      p.part |= vv[u] << u;
    }
  };
  float m = -INFINITY, ssum = 0.f;
  f32x4 acc[4];
  auto process = [&](int i, const Pend& cur) {
    if (i % ngroups == 0) {
      m = -INFINITY;
      ssum = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      // A rank whose LSE is -inf (or NaN, without counts) adds nothing.
      const float lu = (cur.part >> u) & 1 ? cur.l[u] : -INFINITY;
      const float mn = fmaxf(m, lu);
      if (lu > -INFINITY && mn > -INFINITY) {
        const float c_old = m == -INFINITY ? 0.f : fast_exp2((m - mn) * kLog2e);
        const float c_new = fast_exp2((lu - mn) * kLog2e);
        axpy16<kF32>(acc, c_old, cur.x[u], c_new);
        ssum = ssum * c_old + c_new;
        m = mn;
      }
    }
    if (i % ngroups != ngroups - 1) return;     // more ranks of this token to come
    const int t = item_t(i);
    const float inv = ssum > 0.f ? 1.f / ssum : 0.f;
    const size_t row0 = (size_t)t * a.H + h0;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.out + row0 * kLatent), (short)0, kMergeHeads * kLatent * 2, kBufFlags);
    const uint32_t ow = hok ? (uint32_t)(hl * kLatent * 2 + 2 * d0) : kOffNone;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{pack_bf16x2(acc[2 * k][0] * inv, acc[2 * k][1] * inv),
                pack_bf16x2(acc[2 * k][2] * inv, acc[2 * k][3] * inv),
                pack_bf16x2(acc[2 * k + 1][0] * inv, acc[2 * k + 1][1] * inv),
                pack_bf16x2(acc[2 * k + 1][2] * inv, acc[2 * k + 1][3] * inv)},
          rw, ow + 16 * k, 0, 0);
    if (a.out_lse) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.out_lse + row0), (short)0, kMergeHeads * 4, kBufFlags);
      const float lse_v = ssum > 0.f ? m + fast_log2(ssum) * kLn2 : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_v), rs,
                                            hok && (threadIdx.x & 31) == 0 ? (uint32_t)(hl * 4) : kOffNone, 0, 0);
    }
  };
  Pend b0, b1, b2;
  int vv[R];
  load_valid(0, vv);
  load_data(0, vv, b0);
  load_valid(1, vv);
  load_data(1, vv, b1);
  load_valid(2, vv);
  auto step = [&](int i, const Pend& cur, Pend& dst) {
    load_data(i + 2, vv, dst);        // past the last item: no lane reads anything
    load_valid(i + 3, vv);
    process(i, cur);
  };
  for (int i = 0; i < nitems; i += 3) {
    step(i, b0, b2);
    if (i + 1 >= nitems) break;
    step(i + 1, b1, b0);
    if (i + 2 >= nitems) break;
    step(i + 2, b2, b1);
  }
}

// ---------------------------------------------------------------------------
// Merge fused with W_UV.  Workgroup = (head h, a contiguous range of tokens),
// 512 threads.  W_UV[h] (512 x 128 bf16, 128 KiB) is staged once into LDS; the
// tokens then stream through in blocks of 16: the merged latent rows of a
// block (exact LSE-weighted combine of the participating ranks, rounded to
// bf16) go to LDS, and y[tok][n] = o[tok][k] W[k][n] runs on MFMA 16x16x32
// (wave w: n = 16w .. 16w+15), A = o from LDS, B = W: the wave's 16 columns
// of W_UV[h] are read once from the staged copy (transposed LDS reads) and stay
// in registers for the whole launch, so per block only the merged rows are
// read from LDS (keeping B in registers cut the exchange pack's time by a third
// and the fused merge's by 9 %).  Each thread merges one token's 16 dims, so
// three items' partials fit in its registers: two items are always in flight
// while one is merged and projected, and their valid counts come one item
// earlier through scalar loads (a wait for a count never waits for partials).
//
// LDS layouts (both swizzled so that the MFMA operand reads are conflict-free):
//   W  row k (256 B) holds element n at byte (2n) ^ (32 * (k & 7));
//   o  row t (1 KiB) holds 16-byte chunk c at chunk position c ^ (t & 7).
// ---------------------------------------------------------------------------
constexpr int kProjBlk = 16;                       // tokens per block
constexpr int kProjThreads = 512;
constexpr int kWBytes = kLatent * kVHead * 2;      // 128 KiB

// kOne (W = 1): the merge is the identity, and an item's slots are
// consecutive token blocks of the one partial instead of ranks of one block,
// so that more bytes are in flight per item.  An item has two slots with bf16
// partials and one with fp32 partials (kF32: the same bytes); with W_UV's
// operands held in registers more slots no longer fit (measured: three slots
// 14 % slower than two for the pack).
template <bool kValid, bool kOne, bool kF32>
__global__ __launch_bounds__(kProjThreads, 1) void merge_v_up_kernel(const MergeParams a) {
  constexpr int kSlots = kF32 ? 1 : 2;
  constexpr int kWords = kF32 ? 4 : 2;               // 16-byte loads per 16 values
  constexpr int kElem = kF32 ? 4 : 2;                // bytes per partial value
  const uint8_t* outs = kF32 ? (const uint8_t*)a.outs_f : (const uint8_t*)a.outs;
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[kWBytes];
  // Merged rows of a block, two buffers in turn (W_UV and both fill the 160 KiB).
  __shared__ __attribute__((aligned(16))) uint8_t o_buf[2][kProjBlk * kLatent * 2];

  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int per = (a.T + (int)gridDim.y - 1) / (int)gridDim.y;
  const int t_begin = (int)blockIdx.y * per;
  const int t_end = min(a.T, t_begin + per);
  if (t_begin >= t_end) return;

  // Stage W_UV[h]: 128 loads of 1 KiB (4 rows each); wave wv issues 16 of them.
  {
    const uint8_t* src = (const uint8_t*)(a.wuv + (size_t)h * kLatent * kVHead);
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int blk = 16 * wv + i;
      const int o = 1024 * blk + 16 * lane;          // LDS byte
      const int k = o >> 8;
      const int c = o & 255;
      dma_16B_to_lds(src + k * 256 + (c ^ (32 * (k & 7))), w_lds + 1024 * blk);
    }
  }

  // Merge role: thread (token tt = tid / 32 of the block, dims 16*(tid % 32) .. +16);
  // wave wv holds tokens 2wv and 2wv + 1.
  const int tt = threadIdx.x >> 5;
  const int d0 = 16 * (threadIdx.x & 31);
  const size_t plane = (size_t)a.T * a.H;
  // MFMA role: lane (row lr = lane % 16, group g = lane / 16).
  const int lr = lane & 15;
  const int g = lane >> 4;

  // The thread's work is a sequence of items (block b, ranks w0 .. w0+kSlots-1)
  // with w0 = kSlots * j, j < ngroups.
  const int ngroups = kOne ? 1 : (a.W + kSlots - 1) / kSlots;
  const int nblocks = (t_end - t_begin + kProjBlk - 1) / kProjBlk;
  const int nitems = kOne ? (nblocks + kSlots - 1) / kSlots : nblocks * ngroups;
  auto item_tb = [&](int i) { return t_begin + (i / ngroups) * kProjBlk; };
  auto item_w0 = [&](int i) { return kSlots * (i % ngroups); };
  // Slot u of item i: its first token, its rank and whether it exists.
  auto slot_tb = [&](int i, int u) { return kOne ? t_begin + (kSlots * i + u) * kProjBlk : item_tb(i); };
  auto slot_w = [&](int i, int u) { return kOne ? 0 : min(item_w0(i) + u, a.W - 1); };
  auto slot_ok = [&](int i, int u) { return kOne ? slot_tb(i, u) < t_end : item_w0(i) + u < a.W; };
  struct Pend {
    u32x4 x[kSlots][kWords];
    float l[kSlots];
    int part;          // bit u: rank w0 + u was read for this lane
  };
  // Participation of the item's ranks for the thread's token.  With counts, the
  // counts of the wave's two tokens come through scalar loads and ranks that do
  // not take part are not read; without counts every rank's row is read and
  // its LSE decides.
  auto load_valid = [&](int i, int (&vv)[kSlots]) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int tb = slot_tb(i, u);
      const int t = tb + tt;
      const int w = slot_w(i, u);
      if (kValid) {
        const __attribute__((address_space(4))) int32_t* vrow =
            (const __attribute__((address_space(4))) int32_t*)a.valid + (size_t)w * a.T;
        const int c0 = vrow[min(tb + 2 * wv, a.T - 1)];
        const int c1 = vrow[min(tb + 2 * wv + 1, a.T - 1)];
        vv[u] = (lane < 32 ? c0 : c1) > 0 ? 1 : 0;
      } else {
        vv[u] = 1;
      }
      vv[u] &= (i < nitems && slot_ok(i, u) && t < t_end) ? 1 : 0;
    }
  };
  // Every load of an item is issued whether or not the item exists or its lane
  // takes part: buffer loads whose offset lies past the buffer's range return
  // zero without touching memory.  So the number of loads in flight never
  // depends on the data and the compiler's waits stay exact.
  auto load_data = [&](int i, const int (&vv)[kSlots], Pend& p) {
    p.part = 0;
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int tb = min(slot_tb(i, u), a.T - 1);
      const int w = slot_w(i, u);
      const size_t row0 = w * plane + (size_t)tb * a.H + h;     // the block's first token
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(outs + row0 * kLatent * kElem), (short)0, kProjBlk * a.H * kLatent * kElem, kBufFlags);
      const __amdgpu_buffer_rsrc_t rl =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.lses + row0), (short)0, kProjBlk * a.H * 4, kBufFlags);
      const uint32_t oo = vv[u] ? (uint32_t)(tt * a.H * kLatent * kElem + kElem * d0) : kOffNone;
      const uint32_t ol = vv[u] ? (uint32_t)(tt * a.H * 4) : kOffNone;
      p.l[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, ol, 0, 0));
#pragma unroll
      for (int k = 0; k < kWords; ++k) p.x[u][k] = __builtin_amdgcn_raw_buffer_load_b128(ro, oo + 16 * k, 0, 0);
      p.part |= vv[u] << u;
    }
  };

  // B operands (W_UV[h] columns n0 + lr, k = 32s + 8g .. +8) of this wave,
  // read from the staged copy at the first block: source lane j of read r
  // addresses row k = 32s + 8g + 4r + (j >> 2), columns n0 + 4(j & 3) .. +4.
  bf16x8 bw[kLatent / 32];
  bool bw_ready = false;
  auto load_bw = [&]() {
    const int n0 = 16 * wv;
#pragma unroll
    for (int s = 0; s < kLatent / 32; ++s) {
      s16x4 half[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int k = 32 * s + 8 * g + 4 * r + (lr >> 2);
        const int cb = 2 * (n0 + 4 * (lr & 3));
        half[r] = lds_read_tr16_at(w_lds + k * 256 + (cb ^ (32 * (k & 7))));
      }
      bw[s] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  float m = -INFINITY, ssum = 0.f;
  f32x4 acc[4];
  // One item: merge its ranks into the running (m, ssum, acc); after the last
  // rank group of a block, project the block's merged rows.
  // Project the block starting at token tb from the merged rows (acc, m, ssum).
  int nemit = 0;                      // blocks emitted so far (uniform)
  auto emit = [&](int tb) {
    const int t = tb + tt;
    // Buffer nemit & 1: the barrier below, which every wave passes only after
    // its reads of the previous block, makes the buffer of two blocks ago free.
    uint8_t* o_lds = o_buf[nemit & 1];
    ++nemit;
    // Output row of (token tb, head h): slice h / hs holds [T][hs] rows.
    const size_t out_row0 = ((size_t)(h / a.hs) * a.T + tb) * a.hs + h % a.hs;
    // Merged latent row (bf16) into o_lds; an absent token or a row with no
    // participating rank is zero.
    const float inv = ssum > 0.f ? 1.f / ssum : 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = (d0 >> 3) + k;
      *(u32x4*)(o_lds + tt * 1024 + 16 * (c ^ (tt & 7))) =
          u32x4{pack_bf16x2(acc[2 * k][0] * inv, acc[2 * k][1] * inv),
                pack_bf16x2(acc[2 * k][2] * inv, acc[2 * k][3] * inv),
                pack_bf16x2(acc[2 * k + 1][0] * inv, acc[2 * k + 1][1] * inv),
                pack_bf16x2(acc[2 * k + 1][2] * inv, acc[2 * k + 1][3] * inv)};
    }
    if (a.out_lse) {
      // (uniform branch: a kernel argument)
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.out_lse + out_row0), (short)0, kProjBlk * a.hs * 4, kBufFlags);
      const float lse_v = ssum > 0.f ? m + fast_log2(ssum) * kLn2 : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_v), rs,
                                            (threadIdx.x & 31) == 0 && t < t_end ? (uint32_t)(tt * a.hs * 4) : kOffNone, 0, 0);
    }
    // W_UV staged (first block: every load issued so far has landed) and the
    // block's rows written; later items' partial loads may still be in flight
    // (they target registers, not LDS).
    if (tb == t_begin) __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (!bw_ready) {                  // (uniform) W_UV has landed: its operands into registers
      load_bw();
      bw_ready = true;
    }

    // ---- y[tok][n] for the block's 16 tokens, n = 16wv .. 16wv+15 ----
    f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
    const int n0 = 16 * wv;
#pragma unroll
    for (int s = 0; s < kLatent / 32; ++s) {
      // A = o: lane (token lr, group g) takes dims 32s + 8g .. +8 (chunk 4s + g).
      const bf16x8 av = *(const bf16x8*)(o_lds + lr * 1024 + 16 * ((4 * s + g) ^ (lr & 7)));
      // B = W: lane (column n = n0 + lr, group g) holds k = 32s + 8g .. +8.
      y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw[s], y, 0, 0, 0);
    }
    // D: lane (column n = n0 + lr, group g) holds tokens 4g .. 4g+3 of the block.
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.out + out_row0 * kVHead), (short)0, kProjBlk * a.hs * kVHead * 2, kBufFlags);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = 4 * g + r;
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)y[r]), ry,
                                            tb + tk < t_end ? (uint32_t)((tk * a.hs * kVHead + n0 + lr) * 2) : kOffNone, 0, 0);
    }
  };
  auto process = [&](int i, const Pend& cur) {
    if constexpr (kOne) {
      // Each slot is a block of its own; the one partial is its merged row
      // (weight exp(lse - lse) = 1), or zero with LSE -inf if it takes no part.
#pragma unroll
      for (int u = 0; u < kSlots; ++u) {
        const int tb = slot_tb(i, u);
        if (tb >= t_end) break;                       // uniform: depends on i and u only
        const bool in = ((cur.part >> u) & 1) && cur.l[u] > -INFINITY;
        m = in ? cur.l[u] : -INFINITY;
        ssum = in ? 1.f : 0.f;
        f32x4 v[4];
        unpack16<kF32>(cur.x[u], v);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = in ? v[k] : f32x4{0.f, 0.f, 0.f, 0.f};
        emit(tb);
      }
      return;
    } else {
    if (i % ngroups == 0) {
        m = -INFINITY;
        ssum = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kSlots; ++u) {
        const float lu = (cur.part >> u) & 1 ? cur.l[u] : -INFINITY;
        const float mn = fmaxf(m, lu);
        if (lu > -INFINITY && mn > -INFINITY) {
          const float c_old = m == -INFINITY ? 0.f : fast_exp2((m - mn) * kLog2e);
          const float c_new = fast_exp2((lu - mn) * kLog2e);
          axpy16<kF32>(acc, c_old, cur.x[u], c_new);
          ssum = ssum * c_old + c_new;
          m = mn;
        }
      }
      if (i % ngroups != ngroups - 1) return;     // more ranks of this block to come
      emit(item_tb(i));
    }
  };

  // Three register buffers in rotation: while item i is merged, the partials of
  // items i + 1 and i + 2 are in flight (and the counts of item i + 3).  The
  // buffers are never copied (a copy would wait for its loads).
  Pend b0, b1, b2;
  int vv[kSlots];
  load_valid(0, vv);
  load_data(0, vv, b0);
  load_valid(1, vv);
  load_data(1, vv, b1);
  load_valid(2, vv);
  auto step = [&](int i, const Pend& cur, Pend& dst) {
    load_data(i + 2, vv, dst);        // past the last item: no lane reads anything
    load_valid(i + 3, vv);
    process(i, cur);
  };
  for (int i = 0; i < nitems; i += 3) {
    step(i, b0, b2);
    if (i + 1 >= nitems) break;
    step(i + 1, b1, b0);
    if (i + 2 >= nitems) break;
    step(i + 2, b2, b1);
  }
}

hipError_t launch_lse_merge(const MergeParams& p, hipStream_t stream) {
  if (p.T <= 0) return hipSuccess;
  // Ranges of 16 tokens (measured best against 4, 8 and 32 at the DCP4 and
  // DCP8 shapes), shorter when that leaves fewer than 256 workgroups; heads
  // fastest.
  const int hblocks = (p.H + kMergeHeads - 1) / kMergeHeads;
  int ranges = (p.T + 15) / 16;
  const int want = (256 + hblocks - 1) / hblocks;
  if (ranges < want) ranges = want < (p.T + 3) / 4 ? want : (p.T + 3) / 4;
  const dim3 grid((unsigned)hblocks, (unsigned)ranges);
  const bool f32 = p.outs_f != nullptr;
  if (p.W <= 8) {
    if (f32) {
      if (p.valid) hipLaunchKernelGGL((lse_merge_kernel<2, true, true>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((lse_merge_kernel<2, false, true>), grid, dim3(256), 0, stream, p);
    } else {
      if (p.valid) hipLaunchKernelGGL((lse_merge_kernel<4, true, false>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((lse_merge_kernel<4, false, false>), grid, dim3(256), 0, stream, p);
    }
  } else {
    if (f32) {
      if (p.valid) hipLaunchKernelGGL((lse_merge_kernel<4, true, true>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((lse_merge_kernel<4, false, true>), grid, dim3(256), 0, stream, p);
    } else {
      if (p.valid) hipLaunchKernelGGL((lse_merge_kernel<8, true, false>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((lse_merge_kernel<8, false, false>), grid, dim3(256), 0, stream, p);
    }
  }
  return hipGetLastError();
}

hipError_t launch_merge_v_up(const MergeParams& p, hipStream_t stream) {
  if (p.T <= 0) return hipSuccess;
  // About 256 workgroups (one per CU): heads x token ranges.
  int groups = (256 + p.H - 1) / p.H;
  const int max_groups = (p.T + kProjBlk - 1) / kProjBlk;
  if (groups > max_groups) groups = max_groups;
  const dim3 grid((unsigned)p.H, (unsigned)groups);
  const dim3 block(kProjThreads);
  const bool f32 = p.outs_f != nullptr;
  if (p.W == 1) {
    if (f32) {
      if (p.valid) hipLaunchKernelGGL((merge_v_up_kernel<true, true, true>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((merge_v_up_kernel<false, true, true>), grid, block, 0, stream, p);
    } else {
      if (p.valid) hipLaunchKernelGGL((merge_v_up_kernel<true, true, false>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((merge_v_up_kernel<false, true, false>), grid, block, 0, stream, p);
    }
  } else {
    if (f32) {
      if (p.valid) hipLaunchKernelGGL((merge_v_up_kernel<true, false, true>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((merge_v_up_kernel<false, false, true>), grid, block, 0, stream, p);
    } else {
      if (p.valid) hipLaunchKernelGGL((merge_v_up_kernel<true, false, false>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((merge_v_up_kernel<false, false, false>), grid, block, 0, stream, p);
    }
  }
  return hipGetLastError();
}


// Combine of the projected slices a rank receives in the exchange of the merge:
// for every row (token, head of the slice) the W sources' 128-value rows are
// merged by their LSEs (online, sources in order); a source whose LSE is -inf
// (an empty row, as the pack sends it) takes no part.  Thread = (row, 8 values):
// 16 threads per row, 16 rows per workgroup; the sources' loads go out together,
// eight at a time.
__global__ __launch_bounds__(256) void slice_combine_kernel(const SliceParams a) {
  const int row = (int)blockIdx.x * 16 + (int)(threadIdx.x >> 4);
  if (row >= a.rows) return;
  const int d0 = 8 * (threadIdx.x & 15);
  float m = -INFINITY, ssum = 0.f;
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int w0 = 0; w0 < a.W; w0 += 8) {
    float l[8];
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int w = min(w0 + u, a.W - 1);
      l[u] = a.lse[(int64_t)w * a.lse_stride + row];
      x[u] = *(const u32x4*)(a.y + (int64_t)w * a.y_stride + (int64_t)row * kVHead + d0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float lu = w0 + u < a.W ? l[u] : -INFINITY;
      if (lu > -INFINITY) {
        const float mn = fmaxf(m, lu);
        const float c_old = m == -INFINITY ? 0.f : fast_exp2((m - mn) * kLog2e);
        const float c_new = fast_exp2((lu - mn) * kLog2e);
        acc0 = acc0 * c_old + f32x4{bf16_lo(x[u][0]), bf16_hi(x[u][0]), bf16_lo(x[u][1]), bf16_hi(x[u][1])} * c_new;
        acc1 = acc1 * c_old + f32x4{bf16_lo(x[u][2]), bf16_hi(x[u][2]), bf16_lo(x[u][3]), bf16_hi(x[u][3])} * c_new;
        ssum = ssum * c_old + c_new;
        m = mn;
      }
    }
  }
  const float inv = ssum > 0.f ? 1.f / ssum : 0.f;
  *(u32x4*)(a.out + (int64_t)row * kVHead + d0) =
      u32x4{pack_bf16x2(acc0[0] * inv, acc0[1] * inv), pack_bf16x2(acc0[2] * inv, acc0[3] * inv),
            pack_bf16x2(acc1[0] * inv, acc1[1] * inv), pack_bf16x2(acc1[2] * inv, acc1[3] * inv)};
  if (a.out_lse && (threadIdx.x & 15) == 0) a.out_lse[row] = ssum > 0.f ? m + fast_log2(ssum) * kLn2 : -INFINITY;
}

hipError_t launch_slice_combine(const SliceParams& p, hipStream_t stream) {
  if (p.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(slice_combine_kernel, dim3((unsigned)((p.rows + 15) / 16)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla

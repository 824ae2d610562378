// Absorbed-MLA decode for 128 heads on gfx950 (CDNA4): the MFMA-bound case.
//
// What is computed is the same as in mla_decode.hip ("flashattn_mla" API page,
// _forward_decode; PR #24453 review thread for the per-row, per-rank
// seqlen_k).  This file holds the kernel for H = 128 (and H = 64, one head
// block per row), where every cache row is used by 64 or 128 heads of every
// query row and the contraction dominates (about 240 flop per cache byte per
// query row at 128 heads).
//
// Work decomposition.  A workgroup of 8 waves owns one query token, a block of
// 64 heads and one split of the row's visible keys, in 32-key stages.  The
// waves specialise, one of each kind per SIMD:
//   score waves 0..3   wave w computes S^T[key][head] = K Q^T for keys
//                      16(w >> 1) .. +16 of stage k and heads 32(w & 1) .. +32
//                      (MFMA 16x16x32, keys on M, heads on N: one K operand
//                      read from LDS feeds two MFMAs; Q^T resident in VGPRs),
//                      then writes P = 2^(s - m) (bf16, [head][key]) to LDS;
//   PV waves 4..7      wave w accumulates O^T[dim][head] += V^T P^T of stage
//                      k - 1 for latent dims 128(w - 4) .. +128 and all 64
//                      heads (MFMA 32x32x16, V^T from transposed LDS reads,
//                      P^T from LDS).
// So on every SIMD a score wave and a PV wave run side by side, one stage
// apart, with one barrier per stage; P is double-buffered.  The softmax
// reference m of a head is lazy: it only moves when a stage's maximum exceeds
// it by more than 2^16 (always on the first stage), so p <= 2^16.  Every stage
// only tests its scores against m + 16; a stage that fails the test for any
// head takes an extra round before its PV: the two score waves holding a head
// form their halves' maxima from the scores still in their registers, agree
// on the new m through LDS and rewrite P, and the PV waves rescale their
// accumulators.  Stages of 32 rows (36 KiB) arrive by direct-to-LDS loads into
// a 4-slot ring (stages k - 1 and k in use, k + 1 and k + 2 in flight).  The
// PV waves issue and await all stage loads, and the score waves run at a
// higher issue priority: the score waves' chain (K reads, scores, softmax, P
// writes) is the critical path of a stage, so everything else is kept off it.
// The
// two head blocks of a token, and those of the next token (the other query row
// of an MTP request), are consecutive work items placed on the same XCD and
// dispatched back to back, so they share that XCD's L2 for the cache rows.  A
// row split over several workgroups writes fp32 partials that
// combine_fixed_kernel merges afterwards.
#include "mla_common.h"
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXStep = 32;                          // keys per stage
constexpr int kXStageBytes = kXStep * kRowBytes;    // 36 KiB
constexpr int kXBlocks = kXStageBytes / 1024;       // 36 load instructions per stage
constexpr int kXWaves = 8;
constexpr int kXSlots = 4;                          // ring slots
constexpr int kXHeads = 64;                         // heads per workgroup
constexpr int kPRow = 80;                           // LDS bytes per head row of P (64 + 16 pad)
constexpr int kPBuf = kXHeads * kPRow;              // one P buffer
constexpr float kLazyLog2 = 16.f;                   // softmax reference moves past this margin
constexpr int kORow = 272;                          // LDS bytes per staged output row (256 + 16 pad:
                                                    // the 32 heads of one write spread over banks)

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Waits for this wave's loads of stage k: issued after them are, unless k is
// the last stage, the next stage's nine loads.  Only the PV waves load stages.
__device__ __forceinline__ void wait_stage(bool more) {
  if (!more) __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
  else __builtin_amdgcn_s_waitcnt(MLA_VMCNT(9));
}

// LDS writes done, then a workgroup barrier.  (A plain __syncthreads would also
// wait for the ring's loads still in flight.)
// Chunk c of stage row `row` sits at chunk c ^ chunk_swizzle(row) (the low three
// bits only, so a chunk stays in its 128-byte block).  Against the plain row & 7
// this also flips bit 2 when bit 1 of the row is set: the PV waves' transposed
// reads touch four consecutive rows per 16 lanes at two chunk pairs, and with
// row & 7 rows 2i and 2i + 1 of lanes 0..31 land on the same banks (two passes
// instead of one, measured with SQ_LDS_BANK_CONFLICT); the score waves' 16-byte
// reads stay conflict-free either way.
__device__ __forceinline__ int chunk_swizzle(int row) { return (row & 7) ^ ((row << 1) & 4); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// kRuns: the shard layout has runs longer than one token (cp_interleave > 1).
template <bool kPage32, bool kRuns>
__global__ __launch_bounds__(512, 1) void decode_kernel_h128(const DecodeParams a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kXSlots * kXStageBytes];   // 144 KiB
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[2 * kPBuf];              // P, [buf][head][key] bf16
  __shared__ float mx_lds[2][kXHeads];      // per key half: stage max of each head
  __shared__ float alpha_lds[kXHeads];
  __shared__ int bump_lds[2][4];            // [stage parity][score wave]

  // Item = (split, token, head block), head block fastest.  The hardware deals
  // workgroups to the 8 XCDs round-robin by blockIdx and each XCD starts its
  // own in blockIdx order.
  const int hblocks = a.H / kXHeads;
  int item;
  int2 info = int2{-1, 0};                  // {request, the row's local keys} from the order, if known
  if (a.item_map) {
    // Ordered dispatch: grid position p holds the p-th item of the longest-first
    // order.  Groups of four consecutive positions (one request's rows and head
    // blocks) go to one XCD, group g to XCD g mod 8, so every XCD runs its share
    // longest first and a request's workgroups read its cache rows through the
    // same L2.
    const int x = (int)(blockIdx.x & 7), k = (int)(blockIdx.x >> 3);
    const int pos = 4 * (8 * (k >> 2) + x) + (k & 3);
    if (pos >= a.T * hblocks * a.max_splits) return;
    item = a.item_map[pos];
    if (item < 0) return;
    info = a.item_info[pos];
  } else {
    // Item x*per_xcd + k goes to blockIdx 8k + x: consecutive items share an
    // XCD and are dispatched one after the other.
    const int per_xcd = (int)(gridDim.x >> 3);
    item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (item >= a.T * hblocks * a.max_splits) return;
  }
  const int hb = item % hblocks;
  const int t = (item / hblocks) % a.T;
  const int split = item / (hblocks * a.T);
  // The order kernel already located the row; in token order it is found here.
  const RowInfo ri = info.x >= 0 ? RowInfo{info.x, info.y}
                                 : locate_row(a.qsl, a.seq_lens, a.B, t, a.W, a.r, kRuns ? a.I : 1, a.mode);
  const int L = ri.L;
  const int nsplit = num_splits_of(L, a.chunk, a.max_splits);
  if (split >= nsplit) return;
  // The row's key count (with the dispatch order the order kernel wrote it).
  if (a.row_keys && !a.item_map && split == 0 && hb == 0 && threadIdx.x == 0) a.row_keys[t] = L;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h0 = kXHeads * hb;

  if (L == 0) {
    // The row sees no key on this rank: out = 0, lse = -inf (wave w: heads 8w..).
    for (int idx = lane; idx < 8 * 64; idx += 64) {
      const int h = h0 + 8 * w + (idx >> 6);
      zero_out8(a, (size_t)t * a.H + h, 8 * (idx & 63));
      if ((idx & 63) == 0) a.lse[(size_t)t * a.H + h] = -INFINITY;
    }
    return;
  }
  const int j_begin = split * a.chunk;
  const int j_end = split == nsplit - 1 ? L : j_begin + a.chunk;
  const int n_steps = (j_end - j_begin + kXStep - 1) / kXStep;
  const bool scorer = w < 4;

  const int32_t* bt_row = a.bt + (int64_t)ri.b * a.bt_stride;
  const uint8_t* kv_bytes = (const uint8_t*)a.kv;
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring);

  // Stage layout: byte o of a stage is row o / 1152, 16-byte chunk
  // c = (o % 1152) / 16, holding chunk c ^ chunk_swizzle(row) of the row.
  // Keys at or past j_end (a ragged last stage) are clamped to key j_end - 1, a
  // real cached row masked to probability 0.
  auto issue = [&](int i) {
    const int j0 = j_begin + kXStep * i;
    const int slot = i & (kXSlots - 1);
    const uint32_t ldst = ring_lds + slot * kXStageBytes;
    const bool fast = kPage32 && j0 + kXStep <= j_end;
    uint64_t sbase = 0;
    if (fast && w >= 4) {
      // page_size % 32 == 0: the stage's 32 rows are consecutive slots of one page.
      const int pg = a.page_shift >= 0 ? j0 >> a.page_shift : j0 / a.P;
      const int blk = ((const __attribute__((address_space(4))) int32_t*)bt_row)[pg];
      sbase = make_sbase(kv_bytes + ((int64_t)blk * a.kv_bs + (int64_t)(j0 - pg * a.P) * kRow) * 2);
    }
#pragma unroll
    for (int u = 0; u < 9; ++u) {
      if (w < 4) break;                          // PV wave pw loads blocks pw, pw+4, .., pw+32
      const int blkno = (w - 4) + 4 * u;
      const int o = 1024 * blkno + 16 * lane;
      const int row = o / kRowBytes;
      const int cpos = (o - row * kRowBytes) >> 4;
      const uint32_t doff = (uint32_t)(row * kRowBytes + ((cpos ^ chunk_swizzle(row)) << 4));
      if (fast) {
        dma_16B_to_lds_sbase<false>(ldst + 1024 * blkno, doff, sbase);
      } else {
        const int ra = (1024 * blkno) / kRowBytes;   // the block spans rows ra and ra + 1
        const int j = min(j0 + row, j_end - 1);
        const int pa = __builtin_amdgcn_readfirstlane(min(j0 + ra, j_end - 1) / a.P);
        const int pb2 = __builtin_amdgcn_readfirstlane(min(j0 + ra + 1, j_end - 1) / a.P);
        const int ba = ((const __attribute__((address_space(4))) int32_t*)bt_row)[pa];
        const int bb = ((const __attribute__((address_space(4))) int32_t*)bt_row)[pb2];
        const int pg = j / a.P;
        const int64_t rbase = (int64_t)(pg == pa ? ba : bb) * a.kv_bs + (int64_t)(j - pg * a.P) * kRow;
        dma_16B_to_lds(kv_bytes + rbase * 2 + (doff - row * kRowBytes), ring + slot * kXStageBytes + 1024 * blkno);
      }
    }
  };

  // Both roles run the same sequence of barriers: per iteration k the stage
  // barrier, plus a second one when stage k - 1 moved a softmax reference.
  auto stage_barrier = [&](int k) {
    // Stage k's loads have landed (stage k + 1's may be outstanding); the
    // barrier publishes them, the P and maxima of stage k - 1, and tells that
    // every wave is past iteration k - 1, so stage k - 2's slot can take stage
    // k + 2.
    if (w >= 4 && k < n_steps) wait_stage(k + 1 < n_steps);
    asm volatile("s_barrier" ::: "memory");
    if (k + 2 < n_steps) issue(k + 2);
  };
  // Flags of stage k - 1 (double-buffered: stage k's are written meanwhile).
  auto read_flags = [&](int k) {
    const int* f = bump_lds[(k - 1) & 1];
    return k >= 1 ? (f[0] | f[1] | f[2] | f[3]) : 0;
  };
  float* l_lds = (float*)p_lds;              // after the loop: [key half][head] sums
  issue(0);
  if (n_steps > 1) issue(1);

  if (scorer) {
    // ---- score waves: heads 32sg .. +32 (two tiles of 16), keys 16kq .. +16 ----
    // The score waves' chain (scores, softmax, P) sets the pace of a stage;
    // they win issue arbitration over the PV wave on their SIMD.
    __builtin_amdgcn_s_setprio(2);
    const int sg = w & 1;
    const int kq = w >> 1;
    const int qh = lane & 15;
    const int g = lane >> 4;
    bf16x8 q[2][18];                          // Q^T operand per head tile: dims 32s + 8g .. +8
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int hs = h0 + 32 * sg + 16 * ht + qh;
      const uint16_t* qn = a.q_nope + (int64_t)t * a.qn_st + (int64_t)hs * a.qn_sh + 8 * g;
      const uint16_t* qr = a.q_pe + (int64_t)t * a.qp_st + (int64_t)hs * a.qp_sh + 8 * g;
#pragma unroll
      for (int s = 0; s < 16; ++s) q[ht][s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qn + 32 * s));
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x2 v0 = *(const u32x2*)(qr + 32 * s);
        const u32x2 v1 = *(const u32x2*)(qr + 32 * s + 4);
        q[ht][16 + s] = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
      }
    }
    // Score reads: lane (key qh, group g) reads chunk 4s + g of row 16kq + qh:
    // byte row*1152 + 128*(s >> 1) + 16*((4*(s & 1) + g) ^ chunk_swizzle(qh)).
    const uint32_t kbase0 = (16 * kq + qh) * kRowBytes + 16 * (g ^ chunk_swizzle(qh));
    const uint32_t kbase1 = (16 * kq + qh) * kRowBytes + 16 * ((4 + g) ^ chunk_swizzle(qh));
    float m_ref[2] = {-INFINITY, -INFINITY};  // per head tile, of head 32sg + 16ht + qh
    float l_run[2] = {0.f, 0.f};
    float v[2][4];                            // this stage's raw scores, -inf if masked (kept for a redo)
    float thr[2] = {-INFINITY, -INFINITY};    // raw-score test value: (m_ref + margin) / scale
    float psum[2] = {0.f, 0.f};
    auto write_p = [&](int buf) {
      // P rows of heads 32sg + 16ht + qh, keys 16kq + 4g .. +4.
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float base = m_ref[ht] == -INFINITY ? 0.f : m_ref[ht];
        float pe[4];
        psum[ht] = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pe[r] = fast_exp2(fmaf(v[ht][r], a.scale_log2, -base));
          psum[ht] += pe[r];
        }
        uint8_t* prow = p_lds + buf * kPBuf + (32 * sg + 16 * ht + qh) * kPRow + 32 * kq + 8 * g;
        *(u32x2*)prow = u32x2{pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3])};
      }
    };
    // The query loads are done before the first wait counts stage loads only.
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    for (int k = 0; k <= n_steps; ++k) {
      stage_barrier(k);
      // The scores of stage k go out first; the flags of stage k - 1 are read
      // while the MFMAs run.
      const uint8_t* sb = ring + (k & (kXSlots - 1)) * kXStageBytes;
      const int j0 = j_begin + kXStep * k + 16 * kq;     // first key of this wave's half
      f32x4 sc0 = f32x4{0.f, 0.f, 0.f, 0.f}, sc1 = sc0;
      if (k < n_steps) {
        bf16x8 kk[18];
#pragma unroll
        for (int s = 0; s < 18; ++s) kk[s] = *(const bf16x8*)(sb + ((s & 1) ? kbase1 : kbase0) + 128 * (s >> 1));
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          sc0 = mfma_16x16x32(kk[s], q[0][s], sc0);
          sc1 = mfma_16x16x32(kk[s], q[1][s], sc1);
        }
        // Issue order: four K reads ahead, then one further read per two MFMAs
        // (the compiler would otherwise keep only about two reads in flight).
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // LDS reads
#pragma unroll
        for (int i = 0; i < 14; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
      if (read_flags(k)) {
        // A score of stage k - 1 passed its head's reference by more than the
        // margin: the two score waves holding each head publish their halves'
        // maxima of that stage (still in registers), agree on the new reference
        // and rewrite P.
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const float mx = col_max(fmaxf(fmaxf(v[ht][0], v[ht][1]), fmaxf(v[ht][2], v[ht][3]))) * a.scale_log2;
          if (g == 0) mx_lds[kq][32 * sg + 16 * ht + qh] = mx;
        }
        lds_barrier();
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const int hl = 32 * sg + 16 * ht + qh;
          const float mboth = fmaxf(mx_lds[0][hl], mx_lds[1][hl]);
          float alpha = 1.f;
          if (mboth > m_ref[ht] + kLazyLog2) {
            alpha = m_ref[ht] == -INFINITY ? 0.f : fast_exp2(m_ref[ht] - mboth);
            m_ref[ht] = mboth;
            thr[ht] = (mboth + kLazyLog2) / a.scale_log2;
          }
          l_run[ht] *= alpha;
          if (kq == 0 && g == 0) alpha_lds[hl] = alpha;
        }
        write_p((k - 1) & 1);
        lds_barrier();
      }
      if (k >= 1) {
        l_run[0] += psum[0];
        l_run[1] += psum[1];
      }
      if (k < n_steps) {
        // Lane (head qh of tile ht, group g) holds keys j0 + 4g + r.  Only the
        // test against the reference runs every stage; the maxima are formed in
        // the (rare) round that moves a reference.
        bool need = false;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const f32x4 sc = ht ? sc1 : sc0;
          if (j0 + 16 <= j_end) {                 // all 16 keys of the half are visible
#pragma unroll
            for (int r = 0; r < 4; ++r) v[ht][r] = sc[r];
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[ht][r] = (j0 + 4 * g + r < j_end) ? sc[r] : -INFINITY;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) need |= v[ht][r] > thr[ht];
        }
        write_p(k & 1);
        const bool wave_need = (__builtin_amdgcn_read_exec() & __builtin_amdgcn_ballot_w64(need)) != 0;
        if (lane == 0) bump_lds[k & 1][w] = wave_need ? 1 : 0;
      } else if (lane == 0) {
        bump_lds[k & 1][w] = 0;
      }
      // P and flags of stage k are written before the next barrier.
      __builtin_amdgcn_s_waitcnt(MLA_LGKMCNT0);
    }
    // Normalisers through LDS (the P area is free after the barrier).
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const float lsum = col_sum(l_run[ht]);
      if (g == 0) l_lds[kq * kXHeads + 32 * sg + 16 * ht + qh] = lsum;
    }
    __syncthreads();
    if (kq == 0 && g == 0) {
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const int hl = 32 * sg + 16 * ht + qh;
        const float lse_v = (m_ref[ht] + fast_log2(l_lds[hl] + l_lds[kXHeads + hl])) * kLn2;
        const int hs = h0 + hl;
        if (nsplit == 1) a.lse[(size_t)t * a.H + hs] = lse_v;
        else a.ws_lse[((size_t)split * a.T + t) * a.H + hs] = lse_v;
      }
    }
    return;
  }

  // ---- PV waves: dims 128pw .. +128 (four tiles of 32), heads 0..63 ----
  const int pw = w & 3;
  const int hh = lane >> 5;
  const int G = lane >> 4;
  const int jj = lane & 15;
  // V^T (A of O^T = V^T P^T): lane (dim row lane % 32, half hh) needs keys
  // 16m + 8hh + (0..7) of its dim (MFMA m; keys in natural order, as P^T is
  // stored), from two transposed reads per MFMA: within lane group G (hh = G >> 1),
  // source lane j of read r addresses key 16m + 8hh + 4r + (j >> 2) and dims
  // 128pw + 32dt + 16(G & 1) + 4(j & 3): chunk 16pw + 4dt + 2(G & 1) + ((j & 3) >> 1),
  // byte 8(j & 1); the key's low three bits are 4r + (j >> 2).
  uint32_t vb[2][2];                        // [dt & 1][r]; add 128*(dt >> 1)
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int key = 8 * hh + 4 * r + (jj >> 2);
      vb[x][r] = key * kRowBytes + 256 * pw + 16 * ((4 * x + 2 * (G & 1) + ((jj & 3) >> 1)) ^ chunk_swizzle(key)) + 8 * (jj & 1);
    }
  // P^T (B): lane (head 32j + (lane % 32), half hh) reads keys 16m + 8hh .. +8.
  const uint32_t pbase = (uint32_t)((lane & 31) * kPRow + 16 * hh);
  f32x16 o[4][2];                           // O^T tiles [dim tile][head tile]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][j][r] = 0.f;
  for (int k = 0; k <= n_steps; ++k) {
    stage_barrier(k);
    if (read_flags(k)) {
      lds_barrier();                          // the score waves' maxima
      lds_barrier();                          // the score waves' new P and factors
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float al = alpha_lds[32 * j + (lane & 31)];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt][j] *= al;
      }
    }
    if (k >= 1) {
      // PV of stage k - 1: dims 128pw .. +128, all 64 heads, 32 keys.
      const uint8_t* sb = ring + ((k - 1) & (kXSlots - 1)) * kXStageBytes;
      const uint8_t* pb = p_lds + ((k - 1) & 1) * kPBuf + pbase;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 pbv[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) pbv[j] = *(const bf16x8*)(pb + 32 * j * kPRow + 32 * m);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint8_t* vp = sb + 128 * (dt >> 1) + 16 * m * kRowBytes;
          const s16x4 lo = lds_read_tr16_at(vp + vb[dt & 1][0]);
          const s16x4 hi = lds_read_tr16_at(vp + vb[dt & 1][1]);
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int j = 0; j < 2; ++j) o[dt][j] = mfma_32x32x16(va, pbv[j], o[dt][j]);
        }
      }
    }
  }
  __syncthreads();
  __syncthreads();                            // the score waves' sums are in LDS
  // Lane (dim row, half hh) of tile (dt, j) holds head 32j + (lane % 32) and
  // dims 128pw + 32dt + 8q + 4hh + (0..3) in registers 4q .. 4q+3.  A finished
  // row goes out through LDS: stored straight from these registers, a store
  // instruction would touch 32 heads' rows 8 bytes each (measured 8 % slower
  // per call at the MTP shape).
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hl = 32 * j + (lane & 31);
    const float inv = 1.f / (l_lds[hl] + l_lds[kXHeads + hl]);
    const int h = h0 + hl;
    if (nsplit == 1 && !a.out_f) {
      // bf16 row of head hl, this wave's 128 dims, into the (now idle) ring.
      uint8_t* st = ring + pw * (kXHeads * kORow) + hl * kORow + 8 * hh;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *(u32x2*)(st + 2 * (32 * dt + 8 * qd)) =
              u32x2{pack_bf16x2(o[dt][j][4 * qd] * inv, o[dt][j][4 * qd + 1] * inv),
                    pack_bf16x2(o[dt][j][4 * qd + 2] * inv, o[dt][j][4 * qd + 3] * inv)};
    } else {
      // fp32: the row itself (fp32 partials asked for), or the partial of
      // split `split`, read by the combine kernel after this launch.
      float* wp = (nsplit == 1 ? a.out_f + ((size_t)t * a.H + h) * kLatent
                               : a.ws_o + (((size_t)split * a.T + t) * a.H + h) * kLatent) + 128 * pw + 4 * hh;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *(f32x4*)(wp + 32 * dt + 8 * qd) = f32x4{o[dt][j][4 * qd] * inv, o[dt][j][4 * qd + 1] * inv,
                                                   o[dt][j][4 * qd + 2] * inv, o[dt][j][4 * qd + 3] * inv};
    }
  }
  if (nsplit == 1 && !a.out_f) {
    // Each wave reads back its own rows (its LDS writes are complete after the
    // wait) and stores them 256 contiguous bytes per head: lane l takes 16 bytes
    // l % 16 of head 4i + l / 16.
    __builtin_amdgcn_s_waitcnt(MLA_LGKMCNT0);
    const uint8_t* sb = ring + pw * (kXHeads * kORow);
#pragma unroll
    for (int i = 0; i < kXHeads / 4; ++i) {
      const int hr = 4 * i + (lane >> 4);
      const u32x4 v = *(const u32x4*)(sb + hr * kORow + 16 * (lane & 15));
      *(u32x4*)(a.out + ((size_t)t * a.H + h0 + hr) * kLatent + 128 * pw + 8 * (lane & 15)) = v;
    }
  }
}

// Merge of the fixed-size splits of the rows that were split (exact LSE-weighted
// combine, splits in index order).  Workgroup (token t, dim quarter qd, head
// group hg): thread (head 16hg + tid / 16, dims 128qd + 8(tid % 16) .. +8).
__global__ __launch_bounds__(256) void combine_fixed_kernel(const DecodeParams a) {
  const int t = blockIdx.x;
  const RowInfo ri = locate_row(a.qsl, a.seq_lens, a.B, t, a.W, a.r, a.I, a.mode);
  const int np = num_splits_of(ri.L, a.chunk, a.max_splits);
  if (np <= 1) return;
  const int h = 16 * blockIdx.z + (threadIdx.x >> 4);
  if (h >= a.H) return;
  const int d0 = 128 * blockIdx.y + 8 * (threadIdx.x & 15);
  float m = -INFINITY, ssum = 0.f;
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int sp0 = 0; sp0 < np; sp0 += 8) {
    float l[8];
    f32x4 x0[8], x1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = min(sp0 + u, np - 1);
      const size_t srow = ((size_t)sp * a.T + t) * a.H + h;
      l[u] = a.ws_lse[srow];
      const f32x4* src = (const f32x4*)(a.ws_o + srow * kLatent + d0);
      x0[u] = src[0];
      x1[u] = src[1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float mn = fmaxf(m, l[u]);
      if (sp0 + u < np && mn > -INFINITY) {
        const float c_old = m == -INFINITY ? 0.f : fast_exp2((m - mn) * kLog2e);
        const float c_new = fast_exp2((l[u] - mn) * kLog2e);
        acc0 = acc0 * c_old + x0[u] * c_new;
        acc1 = acc1 * c_old + x1[u] * c_new;
        ssum = ssum * c_old + c_new;
        m = mn;
      }
    }
  }
  const float inv = ssum > 0.f ? 1.f / ssum : 0.f;
  const size_t row = (size_t)t * a.H + h;
  store_out8(a, row, d0, acc0 * inv, acc1 * inv);
  if (blockIdx.y == 0 && (threadIdx.x & 15) == 0)
    a.lse[row] = ssum > 0.f ? m + fast_log2(ssum) * kLn2 : -INFINITY;
}

// ---- Longest-first dispatch order ----
//
// Workgroups of the decode grid start in blockIdx order as CUs free up, so the
// order of the items is a list schedule; rows differ several-fold in length
// (and a prefill chunk's rows all belong to one request), so in token order a
// few CUs end up with the longest rows at the end.  Dispatching longest first
// (LPT) bounds the finish spread by the shortest items instead.
//
// Unit = (split s, request b): the rows of b that have keys in split s, with
// both head blocks.  Its length is the number of 32-key stages of its longest
// row (the last one, which sees all Lc_b local keys) in that split.  Units are
// counting-sorted by that length, longest first (equal lengths in any order:
// the order changes only timing, never a result), and expanded into items, a
// unit's rows last row first.  Position p >= the item count maps to -1.
constexpr int kOrdThreads = 1024;
constexpr int kOrdBuckets = 1024;                  // stage counts >= 1023 share the top bucket
constexpr int kOrdMaxUnits = 8192;                 // more (split, request) units: the decode runs unordered
constexpr int kOrdMaxRequests = 4096;              // more requests: likewise
static_assert(kOrdThreads == kOrdBuckets, "one bucket per thread in the order kernel's scan");

struct UnitInfo {
  int q0, rows, first;   // first token, rows with work in this split, index of the first of them
  int stages;            // sort key
};

// Unit u = (split u / B, request u % B), from the request's first token, rows
// and length held in LDS.
__device__ __forceinline__ UnitInfo unit_info(const DecodeParams& a, int u, const int* rq0, const int* rq,
                                              const int* rs) {
  const int s = u / a.B, b = u - s * a.B;
  UnitInfo ui;
  ui.q0 = rq0[b];
  const int Q = rq[b];
  const int S = rs[b];
  const int c = s * a.chunk;
  int cnt;
  if (a.mode == kMaskContext) {
    // Every row sees the same Lx keys: all rows have keys in split s when
    // Lx > c (split 0 keeps them regardless: rows without keys write their
    // empty result).
    const int Lx = shard_count(S - Q, a.W, a.r, a.I);
    ui.first = (s == 0 || Lx > c) ? 0 : Q;
    cnt = min(Lx - c, a.chunk);
  } else {
    // Row i (global position S - Q + i) sees more than c local keys exactly
    // when it sits past the position of local key c, i.e. i >= pos(c) - S + Q.
    // Split 0 also keeps the rows without keys (they write their empty result).
    ui.first = s == 0 ? 0 : max(0, shard_position(c, a.W, a.r, a.I) - S + Q);
    cnt = min(shard_count(S, a.W, a.r, a.I) - c, a.chunk);
  }
  ui.rows = max(0, Q - ui.first);
  ui.stages = ui.rows > 0 && cnt > 0 ? (cnt + kXStep - 1) / kXStep : 0;
  return ui;
}

// Exclusive prefix sum of 64-bit values over the 1024 threads of the
// workgroup: a scan in every wave, then wave 0 scans the 16 wave totals.
__device__ __forceinline__ unsigned long long block_excl_scan64(unsigned long long v, unsigned long long* wsum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  unsigned long long x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  if (wv == 0) {
    const unsigned long long tot = lane < kOrdThreads / 64 ? wsum[lane] : 0ull;
    unsigned long long c = tot;
#pragma unroll
    for (int off = 1; off < kOrdThreads / 64; off <<= 1) {
      const unsigned long long y = __shfl_up(c, off, 64);
      if (lane >= off) c += y;
    }
    if (lane < kOrdThreads / 64) wsum[kOrdThreads / 64 + lane] = c - tot;
  }
  __syncthreads();
  return wsum[kOrdThreads / 64 + wv] + x - v;
}

__global__ __launch_bounds__(kOrdThreads) void h128_order_kernel(const DecodeParams a) {
  // Per bucket (stage count): units in the high 32 bits, their items in the
  // low 32 bits, so that one 64-bit atomic gives a unit both its rank among
  // the sorted units and its first item.
  __shared__ unsigned long long bucket[kOrdBuckets];
  __shared__ int ord[kOrdMaxUnits];      // sorted units
  __shared__ int first_item[kOrdMaxUnits + 1];
  __shared__ int rq0[kOrdMaxRequests], rq[kOrdMaxRequests], rs[kOrdMaxRequests];   // per request
  __shared__ unsigned long long wsum[2 * (kOrdThreads / 64)];   // wave totals, then their exclusive scan
  const int tid = threadIdx.x;
  const int U = a.B * a.max_splits;
  const int hblocks = a.H / kXHeads;
  const int n_map = a.T * hblocks * a.max_splits;
  // The only global reads: every request's first token, rows and length.
  for (int b = tid; b < a.B; b += kOrdThreads) {
    const int q0 = a.qsl[b];
    rq0[b] = q0;
    rq[b] = a.qsl[b + 1] - q0;
    rs[b] = a.seq_lens[b];
  }
  bucket[tid] = 0ull;
  __syncthreads();
  for (int u = tid; u < U; u += kOrdThreads) {
    const UnitInfo ui = unit_info(a, u, rq0, rq, rs);
    atomicAdd(&bucket[min(ui.stages, kOrdBuckets - 1)], (1ull << 32) | (unsigned long long)(ui.rows * hblocks));
  }
  __syncthreads();
  // Longest first: bucket k starts after every unit (and item) of the buckets
  // above it.  Units stay below 2^13 and items below 2^31, so the two halves
  // of the sums never carry into each other.
  const int kb = kOrdBuckets - 1 - tid;
  const unsigned long long cnt = bucket[kb];
  const unsigned long long before = block_excl_scan64(cnt, wsum);
  bucket[kb] = before;
  if (kb == 0) first_item[U] = (int)((before + cnt) & 0xffffffffull);   // the item count
  __syncthreads();
  for (int u = tid; u < U; u += kOrdThreads) {
    const UnitInfo ui = unit_info(a, u, rq0, rq, rs);
    const unsigned long long v =
        atomicAdd(&bucket[min(ui.stages, kOrdBuckets - 1)], (1ull << 32) | (unsigned long long)(ui.rows * hblocks));
    const int rank = (int)(v >> 32);
    ord[rank] = u;
    first_item[rank] = (int)(v & 0xffffffffull);
  }
  __syncthreads();
  const int n_items = first_item[U];
  for (int p = tid; p < n_map; p += kOrdThreads) {
    int item = -1;
    if (p < n_items) {
      // The unit holding item p: the last position whose first item is <= p.
      int lo = 0, hi = U - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first_item[mid] <= p) lo = mid; else hi = mid - 1;
      }
      const int u = ord[lo];
      const int s = u / a.B;
      const UnitInfo ui = unit_info(a, u, rq0, rq, rs);
      const int o = p - first_item[lo];
      const int row = ui.first + ui.rows - 1 - o / hblocks;      // last row first
      item = (s * a.T + ui.q0 + row) * hblocks + o % hblocks;
      const int b = u - s * a.B;
      const int L = row_key_count(rs[b], rq[b], row, a.W, a.r, a.I, a.mode);
      a.item_info[p] = int2{b, L};
      // Every row has exactly one split-0 item of head block 0.
      if (a.row_keys && s == 0 && o % hblocks == 0) a.row_keys[ui.q0 + row] = L;
    }
    a.item_map[p] = item;
  }
}

hipError_t launch_decode_h128(const DecodeParams& p, hipStream_t stream) {
  const int items = p.T * (p.H / kXHeads) * p.max_splits;
  unsigned grid = (unsigned)(((items + 7) / 8) * 8);
  if (p.item_map && (p.B * p.max_splits > kOrdMaxUnits || p.B > kOrdMaxRequests)) {
    DecodeParams q = p;                 // too many units to sort in one workgroup: token order
    q.item_map = nullptr;
    return launch_decode_h128(q, stream);
  }
  if (p.item_map) {
    hipLaunchKernelGGL(h128_order_kernel, dim3(1), dim3(kOrdThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    grid = (unsigned)(((items + 31) / 32) * 32);
  }
  const bool runs = p.I != 1;
  if (p.P % 32 == 0 && !runs) hipLaunchKernelGGL((decode_kernel_h128<true, false>), dim3(grid), dim3(512), 0, stream, p);
  else if (p.P % 32 == 0) hipLaunchKernelGGL((decode_kernel_h128<true, true>), dim3(grid), dim3(512), 0, stream, p);
  else if (!runs) hipLaunchKernelGGL((decode_kernel_h128<false, false>), dim3(grid), dim3(512), 0, stream, p);
  else hipLaunchKernelGGL((decode_kernel_h128<false, true>), dim3(grid), dim3(512), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_splits <= 1) return e;
  hipLaunchKernelGGL(combine_fixed_kernel, dim3((unsigned)p.T, 4, (unsigned)((p.H + 15) / 16)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace mla

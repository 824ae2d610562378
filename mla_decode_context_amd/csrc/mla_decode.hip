// Absorbed-MLA decode over a paged latent cache with the DCP interleaved mask,
// for gfx950 (CDNA4).
//
// What is computed follows the "flashattn_mla" API page (_forward_decode: q_pe
// against k_pe, q_nope against the latent c_kv, c_kv as the value, one softmax
// scale, causal, LSE per token and head) and the PR #24453 review thread (per
// row, per rank seqlen_k under interleaved token placement).
//
// The file holds the decode kernels for every head count except 128 (which
// has its own file), the split combine, the per-row seqlen kernel and a fill.
//
// decode_kernel_h16 (H <= 16, the bandwidth-bound case, about 30 flop per
// cache byte).  One workgroup of four waves per CU; each wave streams its own
// 16-key stages (stage s of a piece belongs to wave s mod 4) from HBM into a
// private two-slot LDS ring with direct-to-LDS loads, the next stage in flight
// while the current one computes, and computes everything for its stages
// alone: the 576-wide scores (MFMA 16x16x32, keys on M, heads on N), the online
// softmax and PV over all 512 latent dims (V^T from transposed LDS reads).
// No barrier in the loop; at the end of a piece the four waves' states merge
// through LDS.  With the balanced schedule (num_splits = 0) the launch's
// rows are cut into equal shares of cache rows per workgroup, computed by every
// wave from seq_lens alone; rows cut at share boundaries become pieces with
// fp32 partials, merged by split_combine_kernel in a second launch.  With a
// fixed split count, each split of a row is one workgroup and the last one to
// finish merges the row (ticket).  An FP8 E4M3 cache stays FP8 in the LDS ring;
// its MFMA operands are converted to bf16 in registers after their LDS reads,
// all of a stage's reads issued at its start (see h16_piece).
//
// decode_kernel (other head counts; 32 heads per workgroup).  Four waves split
// the 576-wide contraction and the 512-wide output: wave w owns latent dims
// 128w .. 128w+127 and rope dims 16w .. 16w+15.  Per 32-key step, the
// workgroup fills a 36 KiB stage of a three-slot ring with direct-to-LDS loads
// (wave w issues nine of its 36 1 KiB loads), every wave forms its partial
// scores over its dims, the four partial score tiles are summed through LDS,
// every wave runs the same online softmax and accumulates PV over its 128
// latent dims.  Split rows merge by ticket as above.
#include "mla_common.h"
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

constexpr int kStep = 32;        // keys per inner step (K of the PV MFMA)
constexpr int kSlab = 128;       // latent dims owned by one wave
constexpr int kStageBytes = kStep * kRowBytes;   // 36 KiB: one step's rows
constexpr int kStages = 3;                        // stages in the LDS ring

// Split rows: the last of the row's pieces to finish merges all partials.
// Every piece has already written its normalised partial and LSE for heads
// h0 .. h0+nheads-1 of token t with device-scope stores.  Partials travel with
// device-scope stores and loads, which write through to and read from the point
// where all XCDs see the same memory, so publishing needs only the wait for this
// workgroup's stores before its ticket -- no write-back of the whole L2 that a
// device-scope fence would cost.  The holder of the last ticket merges (exact
// LSE-weighted combine, pieces in index order whatever the arrival order) and
// puts the counter back to zero for the next call.
__device__ __forceinline__ void ticket_and_merge(const DecodeParams& a, int t, int h0, int nheads,
                                                 int nsplit, SlotMap sm, int counter) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int ticket = __hip_atomic_fetch_add(a.counters + counter, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == nsplit - 1;
  }
  __syncthreads();
  if (!s_last) return;
  // Merge: thread (head hl = tid / 16, dims 32*(tid % 16) .. +32) for each group
  // of 16 heads in turn.  Online LSE combine over the pieces in index order,
  // four pieces' LSEs and partials loaded together per round (each round is a
  // trip to memory: partials are read at device scope).
  const int hl = threadIdx.x >> 4;          // 0..15
  const int d0 = (threadIdx.x & 15) * 32;
  for (int hg = 0; hg < nheads; hg += 16) {
    const int h = h0 + hg + hl;
    if (h < a.H) {
      float m = -INFINITY, ssum = 0.f;
      f32x4 acc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int sp0 = 0; sp0 < nsplit; sp0 += 4) {
        float l[4];
        f32x4 x[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int sp = min(sp0 + u, nsplit - 1);
          const int64_t srow = sm.row(sp) * a.H + h;
          l[u] = load_device(a.ws_lse + srow);
          const float* src = a.ws_o + srow * kLatent + d0;
#pragma unroll
          for (int k = 0; k < 8; ++k) x[u][k] = load_device4(src + 4 * k);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float mn = fmaxf(m, l[u]);
          if (sp0 + u < nsplit && mn > -INFINITY) {
            const float c_old = m == -INFINITY ? 0.f : fast_exp2((m - mn) * kLog2e);
            const float c_new = fast_exp2((l[u] - mn) * kLog2e);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = acc[k] * c_old + x[u][k] * c_new;
            ssum = ssum * c_old + c_new;
            m = mn;
          }
        }
      }
      const float inv = ssum > 0.f ? 1.f / ssum : 0.f;
      const float lse_tot = ssum > 0.f ? m + fast_log2(ssum) * kLn2 : -INFINITY;
      const size_t row = (size_t)t * a.H + h;
#pragma unroll
      for (int k = 0; k < 8; k += 2) store_out8(a, row, d0 + 4 * k, acc[k] * inv, acc[k + 1] * inv);
      if ((threadIdx.x & 15) == 0) a.lse[row] = lse_tot;
    }
  }
  if (threadIdx.x == 0) a.counters[counter] = 0;
}

template <int MT, int NS, bool kPage16>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams a) {
  // One LDS block with a fixed layout: the NS-deep ring of 32-row stages (rows
  // land here straight from HBM) at offset 0, then the double-buffered exchange
  // of partial scores.  The direct-to-LDS loads only ever target the first
  // NS * 36 KiB.
  __shared__ __attribute__((aligned(16))) uint8_t lds_block[NS * kStageBytes + 2 * 4 * 2 * MT * 64 * 16];
  uint8_t (*stage)[kStageBytes] = (uint8_t (*)[kStageBytes])lds_block;
  f32x4 (*sx)[4][2][MT][64] = (f32x4 (*)[4][2][MT][64])(lds_block + NS * kStageBytes);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int g = lane >> 4;

  const int t = blockIdx.x / a.hblocks;
  const int hb = blockIdx.x - t * a.hblocks;
  const int split = blockIdx.y;
  const RowInfo ri = locate_row(a.qsl, a.seq_lens, a.B, t, a.W, a.r, a.I, a.mode);
  const int L = ri.L;
  const int nsplit = num_splits_of(L, a.chunk, (int)gridDim.y);
  if (split >= nsplit) return;
  const int h0 = hb * 16 * MT;
  if (a.row_keys && split == 0 && hb == 0 && threadIdx.x == 0) a.row_keys[t] = L;

  if (L == 0) {
    // The row sees no key on this rank: out = 0, lse = -inf.
    for (int idx = threadIdx.x; idx < 16 * MT * 64; idx += 256) {
      const int h = h0 + (idx >> 6);
      const int c = idx & 63;
      if (h < a.H) {
        zero_out8(a, (size_t)t * a.H + h, c * 8);
        if (c == 0) a.lse[(size_t)t * a.H + h] = -INFINITY;
      }
    }
    return;
  }
  // The last split takes whatever remains, so a row is covered in full even if
  // the grid had fewer splits than ceil(L / chunk).
  const int j_begin = split * a.chunk;
  const int j_end = split == nsplit - 1 ? L : j_begin + a.chunk;
  const int n_steps = (j_end - j_begin + kStep - 1) / kStep;

  // Query operand (B of S^T = K Q^T): lane (head lr, group g) holds, for k-step s,
  // latent dims 128w + 32s + 8g .. +8; for the rope step, groups 0 and 1 hold
  // rope dims 16w + 8g .. +8 and groups 2 and 3 hold zeros (16 rope dims per
  // wave padded to one 32-deep MFMA step).
  bf16x8 qc[MT][4];
  bf16x8 qp[MT];
#pragma unroll
  for (int mu = 0; mu < MT; ++mu) {
    const int h = h0 + 16 * mu + lr;
    if (h < a.H) {
      const uint16_t* qn = a.q_nope + (int64_t)t * a.qn_st + (int64_t)h * a.qn_sh + kSlab * w + 8 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) qc[mu][s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qn + 32 * s));
      const uint16_t* qr = a.q_pe + (int64_t)t * a.qp_st + (int64_t)h * a.qp_sh + 16 * w + 8 * (g & 1);
      const u32x2 q0 = *(const u32x2*)qr;
      const u32x2 q1 = *(const u32x2*)(qr + 4);
      qp[mu] = __builtin_bit_cast(bf16x8, g < 2 ? u32x4{q0[0], q0[1], q1[0], q1[1]} : u32x4{0u, 0u, 0u, 0u});
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qc[mu][s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      qp[mu] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }
  // The q loads must land before the first stage wait counts only stage loads.
  __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));

  const int32_t* bt_row = a.bt + (int64_t)ri.b * a.bt_stride;

  // Stage fill: the 36 KiB stage is 36 blocks of 1 KiB, each written by one
  // direct-to-LDS load instruction (lane l -> bytes 16l .. 16l+15 of the block);
  // wave w issues blocks 9w .. 9w+8.  Byte o of the stage is row o / 1152, 16-byte
  // chunk c = (o % 1152) / 16, which holds chunk c ^ (row & 7) of that cache row.
  // Global addresses of the loads last issued by this wave.  They are kept live
  // (see keep_live below) until the end of the step, so that no instruction
  // writes their registers while the loads may still read them.
  const uint16_t* dma_src[9];
  // Per-lane constants of the stage layout: byte offset of this lane's 16 bytes
  // within 32 consecutive cache rows (row * 1152 + swizzled chunk * 16), and
  // whether the row is in the second half (rows 16..31) of the stage.
  uint32_t lane_off[9];
  bool lane_hi[9];
  int lane_row[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int o = 1024 * (9 * w + i) + 16 * lane;
    const int row = o / kRowBytes;
    const int cpos = (o - row * kRowBytes) >> 4;
    lane_row[i] = row;
    lane_off[i] = (uint32_t)(row * kRowBytes + ((cpos ^ (row & 7)) << 4));
    lane_hi[i] = row >= 16;
  }
  const uint8_t* kv_bytes = (const uint8_t*)a.kv;
  auto issue_stage = [&](int j0, int buf) {
    uint8_t* ldst = stage[buf] + 1024 * 9 * w;
    if (kPage16 && j0 + kStep <= j_end) {
      // Whole stage inside the split and page_size % 16 == 0: rows 0..15 lie in
      // one page and rows 16..31 in one page, so two scalar block-table loads and
      // one 64-bit add per load give every address.
      const int pg0 = j0 / a.P;
      const int pg1 = (j0 + 16) / a.P;
      const int blk0 = load_uniform_i32(bt_row + pg0);
      const int blk1 = load_uniform_i32(bt_row + pg1);
      const uint8_t* base0 = kv_bytes + ((int64_t)blk0 * a.kv_bs + (int64_t)(j0 - pg0 * a.P) * kRow) * 2;
      const uint8_t* base1 = kv_bytes + ((int64_t)blk1 * a.kv_bs + (int64_t)(j0 - pg1 * a.P) * kRow) * 2;
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        dma_src[i] = (const uint16_t*)((lane_hi[i] ? base1 : base0) + lane_off[i]);
        dma_16B_to_lds(dma_src[i], ldst + 1024 * i);
      }
      return;
    }
    // Ragged or trailing stage (or any page size): keys at or past j_end are
    // clamped to j_end - 1 (a real cached row: finite values, masked to
    // probability 0 below), so every path issues the same loads.  A 1 KiB block
    // covers at most two cache rows (ra and ra + 1), so two scalar block-table
    // loads serve each block.
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int ra = (1024 * (9 * w + i)) / kRowBytes;
      const int row = lane_row[i];
      const int j = min(j0 + row, j_end - 1);
      const int pa = __builtin_amdgcn_readfirstlane(min(j0 + ra, j_end - 1) / a.P);
      const int pb2 = __builtin_amdgcn_readfirstlane(min(j0 + ra + 1, j_end - 1) / a.P);
      const int ba = load_uniform_i32(bt_row + pa);
      const int bb = load_uniform_i32(bt_row + pb2);
      const int pg = j / a.P;              // pa or pb2
      const int64_t rbase = (int64_t)(pg == pa ? ba : bb) * a.kv_bs + (int64_t)(j - pg * a.P) * kRow;
      dma_src[i] = (const uint16_t*)(kv_bytes + rbase * 2 + (lane_off[i] - row * kRowBytes));
      dma_16B_to_lds(dma_src[i], ldst + 1024 * i);
    }
  };
  // LDS byte address of 16-byte chunk c of stage row r.
  auto chunk_addr = [&](int r, int c) { return r * kRowBytes + ((c ^ (r & 7)) << 4); };

  float m_run[MT], l_run[MT];
  f32x4 o[8][MT];
#pragma unroll
  for (int mu = 0; mu < MT; ++mu) {
    m_run[mu] = -INFINITY;
    l_run[mu] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt][mu] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Prologue: stages 0 .. NS-2 in flight.
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue_stage(j_begin + kStep * s, s);

  for (int it = 0; it < n_steps; ++it) {
    const int j0 = j_begin + kStep * it;
    const int buf = it % NS;
    // This wave's loads of stage `it` have landed once at most NS-2 newer stages
    // (9 loads each) are outstanding; the barrier then makes every wave's part
    // visible and also tells that all waves are done with the previous step's
    // stage, which the issue below reuses.
    __builtin_amdgcn_s_waitcnt(MLA_VMCNT(9 * (NS - 2)));
    __builtin_amdgcn_s_barrier();
    issue_stage(j0 + kStep * (NS - 1), (it + NS - 1) % NS);
    const uint8_t* sb = stage[buf];

    // Partial scores over this wave's dims: A = keys (lane: key lr of half tau,
    // the same dims as the query operand).
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int r = 16 * tau + lr;
      bf16x8 kc[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) kc[s] = *(const bf16x8*)(sb + chunk_addr(r, 16 * w + 4 * s + g));
      // rope dims 16w + 8g .. +8 (chunk 64 + 2w + g) for groups 0 and 1; the
      // zero query entries of groups 2 and 3 make their key entries irrelevant
      const bf16x8 kp = *(const bf16x8*)(sb + chunk_addr(r, 64 + 2 * w + (g & 1)));
#pragma unroll
      for (int mu = 0; mu < MT; ++mu) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_16x16x32(kc[s], qc[mu][s], acc);
        acc = mfma_16x16x32(kp, qp[mu], acc);
        sx[it & 1][w][tau][mu][lane] = acc;
      }
    }
    __syncthreads();

    // Full scores (fixed summation order, so all waves agree bit for bit),
    // online softmax, and P^T in the B-operand layout: lane (head lr, group g)
    // holds keys 4g..4g+3 (e = 0..3) and 16+4g..16+4g+3 (e = 4..7).
    bf16x8 pb[MT];
#pragma unroll
    for (int mu = 0; mu < MT; ++mu) {
      float v[8];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        f32x4 s4 = sx[it & 1][0][tau][mu][lane];
        s4 += sx[it & 1][1][tau][mu][lane];
        s4 += sx[it & 1][2][tau][mu][lane];
        s4 += sx[it & 1][3][tau][mu][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 16 * tau + 4 * g + r;
          v[tau * 4 + r] = (j < j_end) ? s4[r] * a.scale_log2 : -INFINITY;
        }
      }
      float mx = v[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, v[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[mu], mx);
      const float alpha = fast_exp2(m_run[mu] - m_new);
      m_run[mu] = m_new;
      // The denominator sums the fp32 probabilities; only the PV operand is
      // rounded to bf16 (summing rounded values would cost up to 2^-9 in ln l
      // on rows dominated by one key).
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = fast_exp2(v[e] - m_new);
        pb[mu][e] = (__bf16)pe;
        psum += pe;
      }
      l_run[mu] = l_run[mu] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt][mu] *= alpha;
    }

    // O^T[d][head] += V^T[d][key] P^T[key][head] over this wave's 128 dims; the
    // transposed LDS read gives lane (dim lr, group g) keys 4g..4g+3 (and +16)
    // when source lane lr points at key 4g + (lr >> 2), dims 16dt + 4(lr & 3)..+4.
    const int vr = 4 * g + (lr >> 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int c = 16 * w + 2 * dt + ((lr & 3) >> 1);
      const int off = 8 * (lr & 1);
      const s16x4 lo = lds_read_tr16_at(sb + chunk_addr(vr, c) + off);
      const s16x4 hi = lds_read_tr16_at(sb + chunk_addr(vr + 16, c) + off);
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mu = 0; mu < MT; ++mu) o[dt][mu] = mfma_16x16x32(va, pb[mu], o[dt][mu]);
    }
#pragma unroll
    for (int i = 0; i < 9; ++i) keep_live(dma_src[i]);
  }
  // No stage load may still be writing LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));

  // Finalise: O^T tile (dt, mu) lane (head lr, group g) holds dims
  // 128w + 16dt + 4g + (0..3) of head h0 + 16mu + lr.
#pragma unroll
  for (int mu = 0; mu < MT; ++mu) {
    float lt = l_run[mu];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int h = h0 + 16 * mu + lr;
    if (h >= a.H) continue;
    const float inv = 1.f / lt;
    const float lse_v = (m_run[mu] + fast_log2(lt)) * kLn2;
    if (nsplit == 1) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) store_out4(a, (size_t)t * a.H + h, kSlab * w + 4 * g + 16 * dt, o[dt][mu] * inv);
      if (w == 0 && g == 0) a.lse[(size_t)t * a.H + h] = lse_v;
    } else {
      float* wp = a.ws_o + (((size_t)split * a.T + t) * a.H + h) * kLatent + kSlab * w + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 x = o[dt][mu] * inv;
        store_device(wp + 16 * dt, x[0], x[1]);
        store_device(wp + 16 * dt + 2, x[2], x[3]);
      }
      if (w == 0 && g == 0)
        __hip_atomic_store((uint32_t*)a.ws_lse + ((size_t)split * a.T + t) * a.H + h, __float_as_uint(lse_v),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (nsplit == 1) return;

  ticket_and_merge(a, t, h0, 16 * MT, nsplit, SlotMap{t, a.T, 0}, (int)blockIdx.x);
}

// Up to this many requests the row search runs over a copy of query_start_loc
// in LDS (one coalesced load instead of a chain of dependent global loads).
constexpr int kSeqlensLdsRequests = 4096;

__global__ __launch_bounds__(256) void local_seqlens_kernel(const int32_t* seq_lens, const int32_t* qsl,
                                                            int B, int T, int W, int r, int I, int mode,
                                                            int32_t* row_seqlen, int32_t* shard_len) {
  __shared__ int qsl_lds[kSeqlensLdsRequests + 1];
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (shard_len && i < B) shard_len[i] = shard_count(seq_lens[i], W, r, I);
  if (!row_seqlen) return;
  if (B <= kSeqlensLdsRequests) {
    for (int b = threadIdx.x; b <= B; b += 256) qsl_lds[b] = qsl[b];
    __syncthreads();
    if (i >= T) return;
    int lo = 0, hi = B - 1;                // last b with qsl[b] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (qsl_lds[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int q0 = qsl_lds[lo];
    row_seqlen[i] = row_key_count(seq_lens[lo], qsl_lds[lo + 1] - q0, i - q0, W, r, I, mode);
  } else if (i < T) {
    row_seqlen[i] = locate_row(qsl, seq_lens, B, i, W, r, I, mode).L;
  }
}


// ---------------------------------------------------------------------------
// Decode for up to 16 heads (one 16-head MFMA tile).
//
// With 16 heads the arithmetic is light (about 30 flop per cache byte): the
// kernel exists to keep HBM streaming.  Each of the four waves streams its own
// 16-key stages -- stage s of a piece belongs to wave s mod 4, so the waves
// together sweep 64 consecutive keys (72 KiB) at a time -- into a private
// two-slot LDS ring with direct-to-LDS loads, and computes everything for its
// stages alone: the 576-wide scores, the online softmax and PV over all 512
// latent dims.  The next stage is issued before the current one is awaited,
// and a wave waits only for its own loads: there is no barrier in the loop, so
// one wave's slow load never stalls the others.  At the end of a piece the
// four (max, sum, unnormalised output) states are merged through LDS.
// 144 KiB of LDS: one workgroup per CU.
// ---------------------------------------------------------------------------
constexpr int kWStage = 16;                             // keys per wave stage
constexpr int kWStageBytes = kWStage * kRowBytes;       // 18 KiB
constexpr int kWBlocks = kWStageBytes / 1024;           // 18 load instructions per stage
constexpr int kWRing = 2;                               // slots per wave
constexpr int kWLdsBytes = 4 * kWRing * kWStageBytes;   // 144 KiB

// Writes out = 0 and lse = -inf for heads 0..15 of a row that sees no key.
__device__ __forceinline__ void write_empty_row(const DecodeParams& a, int t) {
  for (int idx = threadIdx.x; idx < 16 * 64; idx += 256) {
    const int h = idx >> 6;
    const int c = idx & 63;
    if (h < a.H) {
      zero_out8(a, (size_t)t * a.H + h, c * 8);
      if (c == 0) a.lse[(size_t)t * a.H + h] = -INFINITY;
    }
  }
}

// One piece of work: local keys [j_begin, j_end) (0 < j_end - j_begin,
// j_begin a multiple of 16) of row t (request b), heads 0..15.  With nsplit == 1
// the piece is the whole row and writes out / lse; otherwise it writes its
// partial to workspace row my_slot and takes part in the row's ticketed merge
// (counter `counter`, slots `sm`).
//
// kFP8: the cache holds FP8 E4M3 codes (576-byte rows, one scale per cache).
// A wave's ring then holds two 9 KiB slots of E4M3 rows, filled by
// direct-to-LDS loads as for bf16 (half the bytes per stage), and the MFMA
// operands are converted in registers right after their LDS reads, with the
// exact E4M3 -> bf16 conversion: a score operand is 8 codes of one key (an
// 8-byte read), a PV operand pair comes from one transposed read of 16-bit
// elements, each element being the codes of two adjacent dims of one key, so
// that the read yields 4 keys of dims 2p and 2p + 1 (split into two operands by
// byte permutes; the O^T tiles 2pt and 2pt + 1 then hold the even and the odd
// dims of dims 32pt .. 32pt + 31).  In a stage row, 16-byte chunk c sits at
// c ^ 2((row >> 2) & 1): the transposed reads are then free of bank conflicts
// (the 8-byte score reads of 16 rows at one column take two passes, the
// 576-byte row stride allows no better).  The cache scale is in the scores'
// exponent factor (scale_log2) and in the final normalisation (out_scale), so
// the conversion adds no rounding.
template <bool kPage16, bool kDeferMerge, bool kFP8>
__device__ __forceinline__ void h16_piece(const DecodeParams& a, uint8_t* lds_block, int t, int b,
                                          int j_begin, int j_end, int nsplit, int64_t my_slot, SlotMap sm,
                                          int counter) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, kept in SGPRs
  const int lr = lane & 15;
  const int g = lane >> 4;
  const int n_stages = (j_end - j_begin + kWStage - 1) / kWStage;
  const int my_n = n_stages > w ? (n_stages - w + 3) / 4 : 0;       // stages w, w+4, w+8, ...

  // Query operand (B of S^T = K Q^T) over all 576 dims: lane (head lr, group g)
  // holds dims 32s + 8g .. +8 for k-step s (s < 16: q_nope, s = 16, 17: q_pe).
  bf16x8 q[18];
  {
    const int h = lr;
    const bool ok = h < a.H;
    const uint16_t* qn = a.q_nope + (int64_t)t * a.qn_st + (int64_t)(ok ? h : 0) * a.qn_sh + 8 * g;
    const uint16_t* qr = a.q_pe + (int64_t)t * a.qp_st + (int64_t)(ok ? h : 0) * a.qp_sh + 8 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const u32x4 v = *(const u32x4*)(qn + 32 * s);
      q[s] = __builtin_bit_cast(bf16x8, ok ? v : u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x2 v0 = *(const u32x2*)(qr + 32 * s);
      const u32x2 v1 = *(const u32x2*)(qr + 32 * s + 4);
      q[16 + s] = __builtin_bit_cast(bf16x8, ok ? u32x4{v0[0], v0[1], v1[0], v1[1]} : u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int32_t* bt_row = a.bt + (int64_t)b * a.bt_stride;
  const uint8_t* kv_bytes = (const uint8_t*)a.kv;
  constexpr int kRowB = kFP8 ? kRow : kRowBytes;           // bytes per cache row
  constexpr int kSlotB = kWStage * kRowB;                  // bytes per ring slot (9 or 18 KiB)
  constexpr int kBlk = kSlotB / 1024;                      // load instructions per stage
  constexpr int kElemB = kFP8 ? 1 : 2;                     // bytes per cache element
  uint8_t* ring = lds_block + w * kWRing * kWStageBytes;   // 36 KiB per wave either way
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring);

  // Stage layout: byte o of the 18 KiB stage is row o / 1152, 16-byte chunk
  // c = (o % 1152) / 16, holding chunk c ^ (row & 7) of that cache row (rows
  // start on the same LDS bank, so eight consecutive rows must use eight
  // different chunks).  Block i (1 KiB) is written by one load: lane l -> bytes
  // 1024i + 16l .. +16, fetched from the byte offset below within the stage's
  // 16 consecutive cache rows.
  // FP8 stages: byte o of the 9 KiB slot is row o / 576, chunk position
  // p = (o % 576) / 16, holding chunk p ^ 2((row >> 2) & 1) of the row.
  uint32_t doff[kBlk];
#pragma unroll
  for (int i2 = 0; i2 < kBlk; ++i2) {
    const int o = 1024 * i2 + 16 * lane;
    const int row = o / kRowB;
    const int cpos = (o - row * kRowB) >> 4;
    doff[i2] = kFP8 ? (uint32_t)(row * kRow + ((cpos ^ (2 * ((row >> 2) & 1))) << 4))
                    : (uint32_t)(row * kRowBytes + ((cpos ^ (row & 7)) << 4));
  }
  // Issue piece stage st into ring slot `slot`.  Keys at or past j_end (the
  // ragged last stage) are clamped to key j_end - 1 -- a real cached row, masked
  // to probability 0 -- so every path issues exactly kBlk loads.
  auto issue = [&](int st, int slot) {
    const int j0 = j_begin + kWStage * st;
    const uint32_t ldst = ring_lds + slot * kSlotB;
    if (kPage16 && j0 + kWStage <= j_end) {
      // page_size % 16 == 0: the stage's 16 rows are consecutive slots of one page.
      const int pg = __builtin_amdgcn_readfirstlane(a.page_shift >= 0 ? j0 >> a.page_shift : j0 / a.P);
      const int blk = load_uniform_i32(bt_row + pg);
      const uint64_t sbase =
          make_sbase(kv_bytes + ((int64_t)blk * a.kv_bs + (int64_t)(j0 - pg * a.P) * kRow) * kElemB);
#pragma unroll
      for (int i2 = 0; i2 < kBlk; ++i2) dma_16B_to_lds_sbase<true>(ldst + 1024 * i2, doff[i2], sbase);
    } else if constexpr (kFP8) {
      // A 1 KiB block spans at most three 576-byte rows, ra .. ra + 2; a lane's
      // 16 bytes lie in one of them.  Keys at or past j_end are clamped as below.
#pragma unroll
      for (int i2 = 0; i2 < kBlk; ++i2) {
        const int o = 1024 * i2 + 16 * lane;
        const int row = o / kRow;
        const int ra = (1024 * i2) / kRow;
        const int j = min(j0 + row, j_end - 1);
        int pgx[3], bx[3];
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          pgx[x] = __builtin_amdgcn_readfirstlane(min(j0 + ra + x, j_end - 1) / a.P);
          bx[x] = load_uniform_i32(bt_row + pgx[x]);
        }
        const int pg = j / a.P;                    // one of pgx[0..2]
        const int blk = pg == pgx[0] ? bx[0] : (pg == pgx[1] ? bx[1] : bx[2]);
        const int64_t rbase = (int64_t)blk * a.kv_bs + (int64_t)(j - pg * a.P) * kRow;
        dma_16B_to_lds_stream(kv_bytes + rbase + (doff[i2] - row * kRow), ring + slot * kSlotB + 1024 * i2);
      }
    } else {
#pragma unroll
      for (int i2 = 0; i2 < kWBlocks; ++i2) {
        const int row = (1024 * i2 + 16 * lane) / kRowBytes;
        const int ra = (1024 * i2) / kRowBytes;     // the block spans rows ra and ra + 1
        const int j = min(j0 + row, j_end - 1);
        const int pa = __builtin_amdgcn_readfirstlane(min(j0 + ra, j_end - 1) / a.P);
        const int pb2 = __builtin_amdgcn_readfirstlane(min(j0 + ra + 1, j_end - 1) / a.P);
        const int ba = load_uniform_i32(bt_row + pa);
        const int bb = load_uniform_i32(bt_row + pb2);
        const int pg = j / a.P;                    // pa or pb2
        const int64_t rbase = (int64_t)(pg == pa ? ba : bb) * a.kv_bs + (int64_t)(j - pg * a.P) * kRow;
        dma_16B_to_lds_stream(kv_bytes + rbase * 2 + (doff[i2] - row * kRowBytes), ring + slot * kWStageBytes + 1024 * i2);
      }
    }
  };
  // Per-lane read bases, so that every read below is a base plus an immediate.
  // Scores: lane (key lr, group g) reads chunk 4s + g of row lr; the swizzle only
  // flips its low three bits, which depend on s through s & 1:
  //   byte = lr*1152 + 128*(s >> 1) + 16*((4*(s & 1) + g) ^ (lr & 7)).
  // PV: source lane (key vr, dims 16dt + 4(lr & 3) ..) reads 8 bytes of chunk
  // 2dt + x, x = (lr & 3) >> 1, at byte 8(lr & 1); its low three bits depend on
  // dt through dt & 3:
  //   byte = vr*1152 + 128*(dt >> 2) + 16*((2*(dt & 3) + x) ^ (vr & 7)) + 8(lr & 1).
  const int k7 = lr & 7;
  const uint32_t kbase0 = lr * kRowBytes + 16 * (g ^ k7);
  const uint32_t kbase1 = lr * kRowBytes + 16 * ((4 + g) ^ k7);
  const int vr = 4 * g + (lr >> 2);
  const int v7 = vr & 7;
  const int vx = (lr & 3) >> 1;
  uint32_t vbase[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) vbase[m] = vr * kRowBytes + 16 * ((2 * m + vx) ^ v7) + 8 * (lr & 1);
  // FP8 reads.  Scores: lane (key lr, group g) reads codes 32s + 8g .. +8 of
  // row lr: chunk 2s + (g >> 1), i.e. byte lr*576 + 32(s ^ b) + 8g with
  // b = (lr >> 2) & 1.  PV: source lane (key vr, pairs 16pt + 4(lr & 3) .. +4)
  // reads 8 bytes at byte vr*576 + 32(pt ^ bv) + 8(lr & 3), bv = (vr >> 2) & 1.
  const int fb = (lr >> 2) & 1, fbv = (vr >> 2) & 1;
  const uint32_t fk0 = lr * kRow + 8 * g + 32 * fb, fk1 = lr * kRow + 8 * g - 32 * fb;   // even / odd s
  const uint32_t fv0 = vr * kRow + 8 * (lr & 3) + 32 * fbv, fv1 = vr * kRow + 8 * (lr & 3) - 32 * fbv;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[32];                    // O^T tiles over all 512 latent dims
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The first stage's loads travel together with the query loads.
  if (my_n > 0) issue(w, 0);
  __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
  for (int k = 0; k < my_n; ++k) {
    const int slot = k & 1;
    // The next stage goes out before this one is awaited.  Its slot was last
    // read by the previous stage, whose LDS reads have all returned
    // (lgkmcnt(0)); only this wave touches its ring, so no barrier is needed.
    if (k + 1 < my_n) {
      __builtin_amdgcn_s_waitcnt(MLA_LGKMCNT0);
      issue(w + 4 * (k + 1), slot ^ 1);
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(kBlk));       // this stage's loads landed, the next one's may not
    } else {
      __builtin_amdgcn_s_waitcnt(MLA_VMCNT(0));
    }
    const uint8_t* sb = ring + slot * kSlotB;
    const int j0 = j_begin + kWStage * (w + 4 * k);

    // S^T[key][head] over 576 dims (A = keys: lane key lr, dims 32s + 8g), two
    // accumulation chains.
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
    // FP8: every LDS read of the stage is issued up front (36 + 32 VGPRs), so
    // that one wave per SIMD waits for LDS once per stage, not once per batch:
    // the 18 score operands, then the 16 transposed V reads, which the softmax
    // does not need.
    u32x2 c8s[kFP8 ? 18 : 1];
    s16x4 vts[kFP8 ? 16 : 1];
    if constexpr (kFP8) {
#pragma unroll
      for (int s = 0; s < 18; ++s) c8s[s] = *(const u32x2*)(sb + ((s & 1) ? fk1 : fk0) + 32 * s);
#pragma unroll
      for (int pt = 0; pt < 16; ++pt) vts[pt] = lds_read_tr16_at(sb + ((pt & 1) ? fv1 : fv0) + 32 * pt);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      bf16x8 kk[9];
#pragma unroll
      for (int u = 0; u < 9; ++u) {
        const int s = 9 * h2 + u;
        if constexpr (kFP8) {
          const u32x2 c8 = c8s[s];
          kk[u] = __builtin_bit_cast(bf16x8, u32x4{fp8x2_to_bf16x2<false>(c8[0]), fp8x2_to_bf16x2<true>(c8[0]),
                                                   fp8x2_to_bf16x2<false>(c8[1]), fp8x2_to_bf16x2<true>(c8[1])});
        } else {
          kk[u] = *(const bf16x8*)(sb + ((s & 1) ? kbase1 : kbase0) + 128 * (s >> 1));
        }
      }
#pragma unroll
      for (int u = 0; u < 9; ++u) {
        const int s = 9 * h2 + u;
        if (s & 1) s1 = mfma_16x16x32(kk[u], q[s], s1);
        else s0 = mfma_16x16x32(kk[u], q[s], s0);
      }
    }
    const f32x4 sc = s0 + s1;

    // Online softmax (base 2).  Lane (head lr, group g) holds keys 4g + r; keys
    // at or past j_end are masked.  The stage always holds a visible key, but a
    // row max of -inf is still kept out of exp2.
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (j0 + 4 * g + r < j_end) ? sc[r] * a.scale_log2 : -INFINITY;
    const float mx = col_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    bf16x8 pb;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pe = fast_exp2(v[r] - m_use);
      pb[r] = (__bf16)pe;
      pb[4 + r] = (__bf16)0.f;
      psum += pe;
    }
    l_run = l_run * alpha + psum;
    // Rescale only when some head's running max moved (once it settles, never).
    if (__builtin_amdgcn_read_exec() & __builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) o[dt] *= alpha;
    }

    // O^T[d][head] += V^T[d][key] P^T[key][head] over all 512 dims; K = 32 with
    // keys 16..31 zero.  The transposed read gives lane (dim lr, group g) keys
    // 4g .. 4g+3 when source lane lr points at key 4g + (lr >> 2), dims
    // 16dt + 4(lr & 3) .. +4.
    if constexpr (kFP8) {
      // Pair tile pt: the transposed read gives lane (pair 16pt + lr, group g)
      // the codes of dims 2p, 2p + 1 of keys 4g .. 4g+3; byte permutes gather
      // the even and the odd dims, which convert to the two operands.
#pragma unroll
      for (int p8 = 0; p8 < 4; ++p8) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int pt = 4 * p8 + u;
          const u32x2 wv = __builtin_bit_cast(u32x2, vts[pt]);
          const uint32_t ev = __builtin_amdgcn_perm(wv[1], wv[0], 0x06040200u);   // keys 0..3, dim 2p
          const uint32_t od = __builtin_amdgcn_perm(wv[1], wv[0], 0x07050301u);   // keys 0..3, dim 2p + 1
          const bf16x8 va0 = __builtin_bit_cast(bf16x8, u32x4{fp8x2_to_bf16x2<false>(ev), fp8x2_to_bf16x2<true>(ev), 0u, 0u});
          const bf16x8 va1 = __builtin_bit_cast(bf16x8, u32x4{fp8x2_to_bf16x2<false>(od), fp8x2_to_bf16x2<true>(od), 0u, 0u});
          o[2 * pt] = mfma_16x16x32(va0, pb, o[2 * pt]);
          o[2 * pt + 1] = mfma_16x16x32(va1, pb, o[2 * pt + 1]);
        }
      }
    } else {
#pragma unroll
    for (int d8 = 0; d8 < 4; ++d8) {
      s16x4 vt[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int dt = 8 * d8 + u;
        vt[u] = lds_read_tr16_at(sb + vbase[dt & 3] + 128 * (dt >> 2));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int dt = 8 * d8 + u;
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vt[u], s16x4{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = mfma_16x16x32(va, pb, o[dt]);
      }
    }
    }
  }
  l_run = col_sum(l_run);

  // Merge of the four waves' states: each stores its (max, sum, output) in LDS
  // (the rings are free once every wave is past its loop), then wave w
  // combines latent dims 128w .. 128w+127 and writes them.
  __syncthreads();
  f32x4* ost = (f32x4*)lds_block;                              // [wave][dt][lane]
  float* mst = (float*)(lds_block + 4 * 32 * 64 * 16);         // [wave][head] max
  float* lst = mst + 64;                                       // [wave][head] sum
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) ost[(w * 32 + dt) * 64 + lane] = o[dt];
  if (g == 0) {
    mst[w * 16 + lr] = m_run;
    lst[w * 16 + lr] = l_run;
  }
  __syncthreads();
  {
    const int h = lr;
    float mv[4], lv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mv[u] = mst[u * 16 + h];
      lv[u] = lst[u * 16 + h];
    }
    const float M = fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3]));   // finite: wave 0 saw a key
    float c[4];
    float Lsum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[u] = mv[u] == -INFINITY ? 0.f : fast_exp2(mv[u] - M);
      Lsum += c[u] * lv[u];
    }
    const float inv = (kFP8 ? a.out_scale : 1.f) / Lsum;
    const float lse_v = (M + fast_log2(Lsum)) * kLn2;
    if (h < a.H) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int dt = 8 * w + i;
        f32x4 x = c[0] * ost[(0 * 32 + dt) * 64 + lane];
#pragma unroll
        for (int u = 1; u < 4; ++u) x += c[u] * ost[(u * 32 + dt) * 64 + lane];
        x *= inv;
        int d = 16 * dt + 4 * g;           // lane holds dims d .. d+3 of head h
        if constexpr (kFP8) {
          // Tiles 2pt, 2pt + 1 hold the even and odd dims 32pt + 8g + 2q (+ 1):
          // tile 2pt writes dims 32pt + 8g .. +4, tile 2pt + 1 dims .. +4 .. +8,
          // after the lanes swap halves with their partner tile's values.
          const int pt = dt >> 1, e = dt & 1;
          f32x4 yy;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // the partner tile's element q, from LDS
            float other = c[0] * ost[(0 * 32 + (dt ^ 1)) * 64 + lane][q];
#pragma unroll
            for (int u = 1; u < 4; ++u) other += c[u] * ost[(u * 32 + (dt ^ 1)) * 64 + lane][q];
            yy[q] = other * inv;
          }
          // dims 32pt + 8g + 4e + r for r = 0..3: element r of the 8-dim run
          // 32pt + 8g + m has m = 4e + r, even m from tile 2pt, odd from 2pt + 1.
          const f32x4 ev = e ? yy : x, od = e ? x : yy;   // tile 2pt, tile 2pt + 1
          x = e ? f32x4{ev[2], od[2], ev[3], od[3]} : f32x4{ev[0], od[0], ev[1], od[1]};
          d = 32 * pt + 8 * g + 4 * e;
        }
        if (nsplit == 1) {
          store_out4(a, (size_t)t * a.H + h, d, x);
        } else if (kDeferMerge) {
          // read by the combine kernel after this launch: plain stores
          *(f32x4*)(a.ws_o + (my_slot * a.H + h) * kLatent + d) = x;
        } else {
          float* wp = a.ws_o + (my_slot * a.H + h) * kLatent + d;
          store_device(wp, x[0], x[1]);
          store_device(wp + 2, x[2], x[3]);
        }
      }
      if (w == 0 && g == 0) {
        if (nsplit == 1)
          a.lse[(size_t)t * a.H + h] = lse_v;
        else if (kDeferMerge)
          a.ws_lse[my_slot * a.H + h] = lse_v;
        else
          __hip_atomic_store((uint32_t*)a.ws_lse + my_slot * a.H + h, __float_as_uint(lse_v),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (nsplit == 1 || kDeferMerge) return;
  ticket_and_merge(a, t, 0, 16, nsplit, sm, counter);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Balanced schedule.  The launch's work is laid out on a line of units: row by
// row in token order, each row takes kRowUnits (its fixed cost: query load,
// pipeline fill, the four-wave merge and the waves' uneven finish; measured, a
// second piece costs a worker about 3.5 stage-times of each wave, and timing
// 10, 14, 18 and 24 units per row put the optimum at 18) followed by one unit
// per 16-key stage.  An FP8 stage takes less time than a bf16 one, so the same
// fixed cost is more of them: 24 units per row (timing 18, 24, 30 and 40).
// Worker g (one workgroup) takes units [g*per, (g+1)*per) with
// per = ceil(total / workers), so every worker streams the same number of cache
// rows (to within one stage) whatever the length mix; a row cut by worker
// boundaries becomes pieces that split_combine_kernel merges after the launch
// (a separate launch spreads that merge over every CU instead of leaving each
// row's pieces to one workgroup at the end).  A worker's
// partial goes to workspace row 2g for the row it continues from its
// predecessor (or that starts exactly on its boundary) and 2g + 1 for the row
// it hands on, so pieces never share a slot.  Every wave computes the schedule
// itself (same inputs, same result), so no barrier is needed.
constexpr int kRowUnits = 18;
constexpr int kRowUnitsFP8 = 24;
constexpr int kMinUnitsPerWorker = 8;

__device__ __forceinline__ int h16_stages(int L) { return (L + kWStage - 1) / kWStage; }

// Units of request b; also returns its first token q0, rows Q and length S.
__device__ __forceinline__ int request_units(const DecodeParams& a, int I, int row_units, int b, int& q0, int& Q,
                                             int& S) {
  q0 = a.qsl[b];
  Q = a.qsl[b + 1] - q0;
  S = a.seq_lens[b];
  int u = 0;
  for (int i = 0; i < Q; ++i) u += row_units + h16_stages(row_key_count(S, Q, i, a.W, a.r, I, a.mode));
  return u;
}

// kRuns: the shard layout has runs longer than one token (cp_interleave > 1);
// without it the run length is the constant 1 and the layout arithmetic folds.
template <bool kPage16, bool kBalanced, bool kRuns, bool kFP8>
__global__ __launch_bounds__(256, 1) void decode_kernel_h16(const DecodeParams a) {
  const int I = kRuns ? a.I : 1;
  constexpr int kRU = kFP8 ? kRowUnitsFP8 : kRowUnits;   // units of a row's fixed cost
  // Four wave rings of two 18 KiB slots; reused for the four-wave merge.
  __shared__ __attribute__((aligned(16))) uint8_t lds_block[kWLdsBytes];

  if constexpr (!kBalanced) {
    // Grid (token, split): split s takes keys [s*chunk, (s+1)*chunk) of the row.
    const int t = blockIdx.x;
    const int split = blockIdx.y;
    const RowInfo ri = locate_row(a.qsl, a.seq_lens, a.B, t, a.W, a.r, I, a.mode);
    const int nsplit = num_splits_of(ri.L, a.chunk, (int)gridDim.y);
    if (split >= nsplit) return;
    if (a.row_keys && split == 0 && threadIdx.x == 0) a.row_keys[t] = ri.L;
    if (ri.L == 0) {
      write_empty_row(a, t);
      return;
    }
    const int j_begin = split * a.chunk;
    const int j_end = split == nsplit - 1 ? ri.L : j_begin + a.chunk;
    h16_piece<kPage16, false, kFP8>(a, lds_block, t, ri.b, j_begin, j_end, nsplit, (int64_t)split * a.T + t,
                              SlotMap{t, a.T, 0}, t);
  } else {
    const int G = (int)gridDim.x;
    const int g = (int)blockIdx.x;
    const int lane = threadIdx.x & 63;
    // Every lane holds one request of the chunk [b0c, b0c + 64): its first
    // token, rows, length and units.  Chunk 0 is kept; the total runs over all.
    int lq0 = 0, lQ = 0, lS = 0;
    const int u_first = lane < a.B ? request_units(a, I, kRU, lane, lq0, lQ, lS) : 0;
    const int inc_first = wave_incl_scan(u_first);
    int total = __shfl(inc_first, 63, 64);
    for (int b0 = 64; b0 < a.B; b0 += 64) {
      const int bb = b0 + lane;
      int x, y, z;
      total += __shfl(wave_incl_scan(bb < a.B ? request_units(a, I, kRU, bb, x, y, z) : 0), 63, 64);
    }
    int per = (total + G - 1) / G;
    if (per < kMinUnitsPerWorker) per = kMinUnitsPerWorker;
    const int x0 = g * per;
    if (x0 >= total) return;
    const int x1 = min(x0 + per, total);
    // The request whose unit range holds x0 (requests without rows own none).
    int b = 0, pos = 0, carry = 0, b0c = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int bb = b0 + lane;
      int u = u_first, inc = inc_first;
      if (b0 > 0) {
        u = bb < a.B ? request_units(a, I, kRU, bb, lq0, lQ, lS) : 0;
        inc = wave_incl_scan(u);
      }
      const bool hit = bb < a.B && carry + inc - u <= x0 && x0 < carry + inc;
      const uint64_t m = __ballot(hit);
      if (m) {
        const int src = __ffsll((unsigned long long)m) - 1;
        b = b0 + src;
        b0c = b0;
        pos = carry + __shfl(inc - u, src, 64);
        break;
      }
      carry += __shfl(inc, 63, 64);
    }
    b = __builtin_amdgcn_readfirstlane(b);
    b0c = __builtin_amdgcn_readfirstlane(b0c);
    pos = __builtin_amdgcn_readfirstlane(pos);
    // Request fields come from the lane that holds them (no memory round trip)
    // while b stays in the cached chunk.
    auto fetch = [&](int bq, int& q0_, int& Q_, int& S_) {
      if (bq - b0c < 64) {
        q0_ = __builtin_amdgcn_readfirstlane(__shfl(lq0, bq - b0c, 64));
        Q_ = __builtin_amdgcn_readfirstlane(__shfl(lQ, bq - b0c, 64));
        S_ = __builtin_amdgcn_readfirstlane(__shfl(lS, bq - b0c, 64));
      } else {
        q0_ = a.qsl[bq];
        Q_ = a.qsl[bq + 1] - q0_;
        S_ = a.seq_lens[bq];
      }
    };
    int q0, Q, S, i = 0;
    fetch(b, q0, Q, S);
    while (pos < x1) {
      if (i == Q) {      // next request; one exists because pos < total
        ++b;
        fetch(b, q0, Q, S);
        i = 0;
        continue;
      }
      const int L = row_key_count(S, Q, i, a.W, a.r, I, a.mode);
      const int n = h16_stages(L);
      const int t = q0 + i;
      if (pos + kRU + n > x0) {
        if (L == 0) {
          if (pos >= x0) {                           // the row's owner is the worker holding its start
            write_empty_row(a, t);
            if (threadIdx.x == 0) {
              a.row_desc[t] = int4{0, 0, 0, 0};
              if (a.row_keys) a.row_keys[t] = 0;
            }
          }
        } else {
          const int s0 = pos + kRU;           // unit of the row's first stage
          const int lo = max(x0 - s0, 0);
          const int hi = min(x1 - s0, n);
          if (lo < hi) {
            const int gf = s0 / per;                 // workers holding the row's stages: gf .. gl
            const int gl = (s0 + n - 1) / per;
            const SlotMap sm{2 * gf, 2, s0 == gf * per ? 0 : 1};
            // The worker of the row's first piece tells the combine kernel how
            // to find the row's pieces.
            if (g == gf && threadIdx.x == 0) {
              a.row_desc[t] = int4{gl - gf + 1, sm.base, sm.adj0, 0};
              if (a.row_keys) a.row_keys[t] = L;
            }
            h16_piece<kPage16, true, kFP8>(a, lds_block, t, b, lo * kWStage, min(hi * kWStage, L), gl - gf + 1,
                                     sm.row(g - gf), sm, t);
            __syncthreads();                         // LDS is reused by the next piece
          }
        }
      }
      pos += kRU + n;
      ++i;
    }
  }
}

// Merge of the pieces of rows that the balanced schedule split (exact LSE-
// weighted combine, pieces in index order).  Workgroup (token t, dim quarter
// qd): thread (head h = tid / 16, dims 128qd + 8(tid % 16) .. +8); rows that
// were not split were finished by the decode kernel.
__global__ __launch_bounds__(256) void split_combine_kernel(const DecodeParams a) {
  const int t = blockIdx.x;
  const int4 desc = a.row_desc[t];
  const int np = desc.x;
  if (np <= 1) return;
  const SlotMap sm{desc.y, 2, desc.z};
  const int h = threadIdx.x >> 4;
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
      const int64_t srow = sm.row(sp) * a.H + h;
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

hipError_t launch_decode(const DecodeParams& p, int mtiles, int max_splits, int workers, hipStream_t stream) {
  const bool page16 = p.P % 16 == 0;
  if (mtiles == 1 && workers > 0) {
    const dim3 grid((unsigned)workers);
    const bool runs = p.I != 1;
    if (p.kv_fp8) {
      if (page16 && !runs) hipLaunchKernelGGL((decode_kernel_h16<true, true, false, true>), grid, dim3(256), 0, stream, p);
      else if (page16) hipLaunchKernelGGL((decode_kernel_h16<true, true, true, true>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((decode_kernel_h16<false, true, true, true>), grid, dim3(256), 0, stream, p);
    } else {
      if (page16 && !runs) hipLaunchKernelGGL((decode_kernel_h16<true, true, false, false>), grid, dim3(256), 0, stream, p);
      else if (page16) hipLaunchKernelGGL((decode_kernel_h16<true, true, true, false>), grid, dim3(256), 0, stream, p);
      else if (!runs) hipLaunchKernelGGL((decode_kernel_h16<false, true, false, false>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((decode_kernel_h16<false, true, true, false>), grid, dim3(256), 0, stream, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(split_combine_kernel, dim3((unsigned)p.T, 4), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(p.T * p.hblocks), (unsigned)max_splits);
  if (mtiles == 1) {
    if (p.kv_fp8) {
      if (page16) hipLaunchKernelGGL((decode_kernel_h16<true, false, true, true>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((decode_kernel_h16<false, false, true, true>), grid, dim3(256), 0, stream, p);
    } else {
      if (page16) hipLaunchKernelGGL((decode_kernel_h16<true, false, true, false>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((decode_kernel_h16<false, false, true, false>), grid, dim3(256), 0, stream, p);
    }
  } else {
    if (page16) hipLaunchKernelGGL((decode_kernel<2, kStages, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_kernel<2, kStages, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_local_seqlens(const int32_t* seq_lens, const int32_t* qsl, int B, int T, int W,
                                int r, int I, int mode, int32_t* row_seqlen, int32_t* shard_len, hipStream_t stream) {
  const int n = T > B ? T : B;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(local_seqlens_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, seq_lens, qsl,
                     B, T, W, r, I, mode, row_seqlen, shard_len);
  return hipGetLastError();
}

}  // namespace mla

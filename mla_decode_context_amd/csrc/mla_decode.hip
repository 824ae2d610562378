// Absorbed-MLA decode over a paged latent cache with the DCP interleaved mask,
// for gfx950 (CDNA4).
//
// What is computed follows the "flashattn_mla" API page (_forward_decode: q_pe
// against k_pe, q_nope against the latent c_kv, c_kv as the value, one softmax
// scale, causal, LSE per token and head) and the PR #24453 review thread (per
// row, per rank seqlen_k under interleaved token placement).
//
// Work decomposition.  One workgroup of 4 wavefronts owns one query token, a
// block of 16*MT heads (the MFMA M dimension) and one split of that row's
// visible local keys.  The four waves split the 576-wide contraction and the
// 512-wide output between them: wave w owns latent dims [128w, 128w+128) and
// rope dims [16w, 16w+16).  Per step of 32 keys:
//   1. each wave loads only its 288 bytes of each of the 32 cache rows straight
//      into registers (block-table indirection per key; the four waves together
//      read every 1152-byte row exactly once);
//   2. partial scores S^T = K Q^T over the wave's dims with MFMA (keys as M=16
//      rows of the A operand, heads as N columns of the B operand);
//   3. the four partial score tiles are summed through LDS;
//   4. every wave runs the same online softmax (base 2, fp32) on the full
//      scores -- masked keys get probability 0 and zeroed values;
//   5. O^T += V^T P^T with MFMA on the wave's own 128 latent dims, where V^T
//      comes from the wave's LDS copy of the rows via the transposed LDS read
//      (ds_read_b64_tr_b16) and P^T is the softmax output already in the
//      B-operand layout.
// The next step's rows are loaded while the current step computes.  When a
// row's keys are split over several workgroups, each writes its normalised
// partial (fp32) and LSE to the workspace and the last one to finish merges
// them (exact LSE-weighted combine) in the same launch.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

constexpr int kStep = 32;        // keys per inner step (K of the PV MFMA)
constexpr int kSlab = 128;       // latent dims owned by one wave
constexpr int kVStride = 144;    // LDS row stride of a wave's value slab (bf16): 288 B

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed 64-bit LDS read: within each 16-lane group, lane i receives
// element (i & 3) of the four-element chunk addressed by lane 4e + (i >> 2),
// for e = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uint16_t*)p);
}

// Splits of a row with L visible keys: ceil(L / chunk), at least 1, at most the
// grid's split extent.
__device__ __forceinline__ int num_splits_of(int L, int chunk, int max_splits) {
  const int n = L > 0 ? (L + chunk - 1) / chunk : 1;
  return n < max_splits ? n : max_splits;
}

template <int MT>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams a) {
  __shared__ __attribute__((aligned(16))) uint16_t vslab[4][kStep * kVStride];
  __shared__ __attribute__((aligned(16))) f32x4 sx[2][4][2][MT][64];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int g = lane >> 4;

  const int t = blockIdx.x / a.hblocks;
  const int hb = blockIdx.x - t * a.hblocks;
  const int split = blockIdx.y;
  const RowInfo ri = locate_row(a.qsl, a.seq_lens, a.B, t, a.W, a.r);
  const int L = ri.L;
  const int nsplit = num_splits_of(L, a.chunk, (int)gridDim.y);
  if (split >= nsplit) return;
  const int h0 = hb * 16 * MT;

  if (L == 0) {
    // The row sees no key on this rank: out = 0, lse = -inf.
    for (int idx = threadIdx.x; idx < 16 * MT * 64; idx += 256) {
      const int h = h0 + (idx >> 6);
      const int c = idx & 63;
      if (h < a.H) {
        *(u32x4*)(a.out + ((size_t)t * a.H + h) * kLatent + c * 8) = u32x4{0u, 0u, 0u, 0u};
        if (c == 0) a.lse[(size_t)t * a.H + h] = -INFINITY;
      }
    }
    return;
  }
  // The last split takes whatever remains, so a row is covered in full even if
  // the grid had fewer splits than ceil(L / chunk).
  const int j_begin = split * a.chunk;
  const int j_end = split == nsplit - 1 ? L : j_begin + a.chunk;

  // Query operand (B of S^T = K Q^T): lane (head lr, group g) holds, for k-step s,
  // latent dims 128w + 32s + 8g .. +8, and rope dims 16w + 4g .. +4.
  bf16x8 qc[MT][4];
  s16x4 qp[MT];
#pragma unroll
  for (int mu = 0; mu < MT; ++mu) {
    const int h = h0 + 16 * mu + lr;
    if (h < a.H) {
      const uint16_t* qn = a.q_nope + (int64_t)t * a.qn_st + (int64_t)h * a.qn_sh + kSlab * w + 8 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) qc[mu][s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qn + 32 * s));
      const uint16_t* qr = a.q_pe + (int64_t)t * a.qp_st + (int64_t)h * a.qp_sh + 16 * w + 4 * g;
      qp[mu] = __builtin_bit_cast(s16x4, *(const u32x2*)qr);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qc[mu][s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      qp[mu] = s16x4{0, 0, 0, 0};
    }
  }

  const int32_t* bt_row = a.bt + (int64_t)ri.b * a.bt_stride;
  // Key operand (A of S^T): lane (key lr of half tau, group g) holds the same dims.
  u32x4 kc[2][4];
  u32x2 kp[2];
  auto load_step = [&](int j0, u32x4 (&c)[2][4], u32x2 (&pr)[2]) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int j = j0 + 16 * tau + lr;
      if (j < j_end) {
        const int blk = bt_row[j / a.P];
        const uint16_t* row = a.kv + (int64_t)blk * a.kv_bs + (int64_t)(j % a.P) * kRow;
#pragma unroll
        for (int s = 0; s < 4; ++s) c[tau][s] = *(const u32x4*)(row + kSlab * w + 32 * s + 8 * g);
        pr[tau] = *(const u32x2*)(row + kLatent + 16 * w + 4 * g);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) c[tau][s] = u32x4{0u, 0u, 0u, 0u};
        pr[tau] = u32x2{0u, 0u};
      }
    }
  };

  float m_run[MT], l_run[MT];
  f32x4 o[8][MT];
#pragma unroll
  for (int mu = 0; mu < MT; ++mu) {
    m_run[mu] = -INFINITY;
    l_run[mu] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt][mu] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint16_t* vs = vslab[w];
  load_step(j_begin, kc, kp);
  int buf = 0;
  for (int j0 = j_begin; j0 < j_end; j0 += kStep) {
    u32x4 nc[2][4];
    u32x2 np[2];
    const bool more = j0 + kStep < j_end;
    if (more) load_step(j0 + kStep, nc, np);

    // This wave's latent slab of the 32 rows -> LDS (read back transposed below).
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        *(u32x4*)(vs + (16 * tau + lr) * kVStride + 32 * s + 8 * g) = kc[tau][s];

    // Partial scores over this wave's dims.
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int mu = 0; mu < MT; ++mu) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_16x16x32(__builtin_bit_cast(bf16x8, kc[tau][s]), qc[mu][s], acc);
        acc = mfma_16x16x16(__builtin_bit_cast(s16x4, kp[tau]), qp[mu], acc);
        sx[buf][w][tau][mu][lane] = acc;
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
        f32x4 s4 = sx[buf][0][tau][mu][lane];
        s4 += sx[buf][1][tau][mu][lane];
        s4 += sx[buf][2][tau][mu][lane];
        s4 += sx[buf][3][tau][mu][lane];
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

    // O^T[d][head] += V^T[d][key] P^T[key][head] over this wave's 128 dims.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* src = vs + (4 * g + (lr >> 2)) * kVStride + 16 * dt + 4 * (lr & 3);
      const s16x4 lo = lds_read_tr16(src);
      const s16x4 hi = lds_read_tr16(src + 16 * kVStride);
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mu = 0; mu < MT; ++mu) o[dt][mu] = mfma_16x16x32(va, pb[mu], o[dt][mu]);
    }

    if (more) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
        for (int s = 0; s < 4; ++s) kc[tau][s] = nc[tau][s];
        kp[tau] = np[tau];
      }
    }
    buf ^= 1;
  }

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
      uint16_t* op = a.out + ((size_t)t * a.H + h) * kLatent + kSlab * w + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 x = o[dt][mu] * inv;
        *(u32x2*)(op + 16 * dt) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      }
      if (w == 0 && g == 0) a.lse[(size_t)t * a.H + h] = lse_v;
    } else {
      float* wp = a.ws_o + (((size_t)split * a.T + t) * a.H + h) * kLatent + kSlab * w + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *(f32x4*)(wp + 16 * dt) = o[dt][mu] * inv;
      if (w == 0 && g == 0) a.ws_lse[((size_t)split * a.T + t) * a.H + h] = lse_v;
    }
  }
  if (nsplit == 1) return;

  // Split rows: the last of the row's splits to finish merges all partials.
  // Each split publishes its partial (release fence), then takes a ticket;
  // the holder of the last ticket acquires and merges, and puts the counter
  // back to zero for the next call.
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int ticket = atomicAdd(a.counters + blockIdx.x, 1);
    s_last = ticket == nsplit - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const size_t plane = (size_t)a.T * a.H;
  for (int hh = w; hh < 16 * MT; hh += 4) {
    const int h = h0 + hh;
    if (h >= a.H) break;
    const size_t row = (size_t)t * a.H + h;
    float mx = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, a.ws_lse[sp * plane + row]);
    float sum = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) sum += fast_exp2((a.ws_lse[sp * plane + row] - mx) * kLog2e);
    const float lse_tot = mx + fast_log2(sum) * kLn2;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < nsplit; ++sp) {
      const float wgt = fast_exp2((a.ws_lse[sp * plane + row] - lse_tot) * kLog2e);
      const float* src = a.ws_o + (sp * plane + row) * kLatent + lane * 8;
      const f32x4 x0 = *(const f32x4*)src;
      const f32x4 x1 = *(const f32x4*)(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += wgt * x0[e];
        acc[4 + e] += wgt * x1[e];
      }
    }
    *(u32x4*)(a.out + row * kLatent + lane * 8) =
        u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    if (lane == 0) a.lse[row] = lse_tot;
  }
  if (threadIdx.x == 0) a.counters[blockIdx.x] = 0;
}

__global__ __launch_bounds__(256) void local_seqlens_kernel(const int32_t* seq_lens, const int32_t* qsl,
                                                            int B, int T, int W, int r,
                                                            int32_t* row_seqlen, int32_t* shard_len) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (row_seqlen && i < T) row_seqlen[i] = locate_row(qsl, seq_lens, B, i, W, r).L;
  if (shard_len && i < B) shard_len[i] = ceil_div_pos(seq_lens[i] - r, W);
}

hipError_t launch_decode(const DecodeParams& p, int mtiles, int max_splits, hipStream_t stream) {
  const dim3 grid((unsigned)(p.T * p.hblocks), (unsigned)max_splits);
  if (mtiles == 1)
    hipLaunchKernelGGL(decode_kernel<1>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_kernel<2>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_local_seqlens(const int32_t* seq_lens, const int32_t* qsl, int B, int T, int W,
                                int r, int32_t* row_seqlen, int32_t* shard_len, hipStream_t stream) {
  const int n = T > B ? T : B;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(local_seqlens_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, seq_lens, qsl,
                     B, T, W, r, row_seqlen, shard_len);
  return hipGetLastError();
}

}  // namespace mla

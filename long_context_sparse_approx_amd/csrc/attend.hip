// Stages 5-6: exact attention over the selected tokens, split-K over chunks.
//
// "FASA: Frequency-aware Sparse Attention", section 3 stage 2 (FAC): full
// precision attention on the selected tokens only, at their original
// positions (the cache holds post-RoPE keys, so positions are kept).
// "Stratified Sparse Attention speeds up decoding 2.96x at 1M context",
// "How SSA stratifies the cache": sampled tokens carry the inverse inclusion
// probability, applied here as the logit bias -log(pi_j) stored with the
// selection.  "S2O: Early Stopping for Sparse Attention via Online
// Permutation", methodology part 3: each split keeps the online-softmax
// state (m, l, acc); the merge resumes from the stored states.
//
// One wavefront per (selection unit, member block, split).  The 16 query
// columns of the tiles hold up to 16 / G members of the unit's query group
// (consecutive query positions) times their G heads, so one pass over the
// selected K/V rows serves them all; column (member t, head) masks the
// positions past its own causal span [0, P - T + t] and keeps its own
// online-softmax state.  A tile is 32 selected tokens; both
// products run on MFMA v_mfma_f32_16x16x32_bf16:
//   QK:  D[16 tokens x 16 heads] = K_tile[16 x 32 dims] * Q^T[32 dims x 16 heads],
//        two halves of 16 tokens, d/32 steps each; query heads beyond the
//        group size are zero rows.
//   PV:  D[16 heads x 16 cols] += P[16 heads x 32 tokens] * V[32 tokens x 16 cols],
//        d/16 steps; P is split into bf16 hi + lo parts (two MFMAs) so the
//        probabilities keep ~16 significant bits.
// Layout choices that remove every LDS transpose:
//   * QK's output D holds (token 4q+r, head n) in lane 16q+n; PV's A operand
//     wants (head n, k-slot 8q+i) in lane 16q+n, so k-slot 8q+i is defined as
//     token 4q+i (i < 4) or 16+4q+(i-4) (i >= 4): P never moves.
//   * PV's output column n of step j is head dim n*(d/16)+j, so lane n's V
//     operand for all steps is one contiguous d/16-element slice of each of
//     its 8 token rows: a wave-wide load reads 4 full 256-byte rows.
#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <int D>
struct VSlice;
template <>
struct VSlice<128> {
  using T = uint4;  // 8 dims
  static __device__ __forceinline__ T zero() { return make_uint4(0u, 0u, 0u, 0u); }
  static __device__ __forceinline__ uint32_t word(const T& v, int w) {
    return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
  }
};
template <>
struct VSlice<64> {
  using T = uint2;  // 4 dims
  static __device__ __forceinline__ T zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ uint32_t word(const T& v, int w) { return w == 0 ? v.x : v.y; }
};

constexpr int kBatch = 256;  // selected items resolved to cache rows at a time

// SPLIT: the keys are held in two arrays of the same row numbering: the
// scored dims (2 * pair_count per row) apart from the others ("FASA:
// Frequency-aware Sparse Attention", section 3, variants: FASA-M keeps the
// dominant key components resident and moves the rest of the key and the
// values elsewhere); a row is put back together from its 16-byte slices.
template <int D, bool SPLIT>
__global__ __launch_bounds__(64) void attend_kernel(AttendArgs a) {
  constexpr int KK = D / 32;   // QK steps over the head dim
  constexpr int DPL = D / 16;  // head dims per PV column = PV steps
  using VS = VSlice<D>;
  __shared__ int rows_sh[kBatch + 32];
  __shared__ float lw_sh[kBatch + 32];
  __shared__ int pos_sh[kBatch + 32];

  const int slot = blockIdx.x;  // partial state written by this wave
  const int s = slot / a.nsub;   // split: a range of chunks
  const int sub = slot - s * a.nsub;  // share of each chunk's items
  const int nslot = a.nsplit * a.nsub;
  const int u = blockIdx.y / a.mblocks;  // selection unit (b, grp, h)
  const int mb = blockIdx.y - u * a.mblocks;
  const int bg = u / a.Hkv;
  const int h = u - bg * a.Hkv;
  const int b = bg / a.NG;
  const int grp = bg - b * a.NG;
  const int t_a = grp * a.g + mb * a.mpw;  // first member of this block
  const int nmem = min(min(a.mpw, (grp + 1) * a.g - t_a), a.T - t_a);
  if (nmem <= 0) return;  // uniform over the wave
  const int lane = threadIdx.x;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int P = clamp_len(a.seq_lens[b], a.max_seq_len);
  // Column n16 = (member t_a + n16 / G, head n16 % G); columns past the
  // block's members have an empty span.
  const bool col_valid = n16 < nmem * a.G;
  const int col_t = t_a + (col_valid ? n16 / a.G : 0);
  const int col_g = col_valid ? n16 - (n16 / a.G) * a.G : 0;
  const int L_col = col_valid ? member_span(P, a.T, col_t) : 0;
  const int L = member_span(P, a.T, t_a + nmem - 1);  // the block's widest span
  const int ncL = (L + kChunk - 1) / kChunk;
  const int c_begin = (int)((int64_t)s * ncL / a.nsplit);
  const int c_end = (int)((int64_t)(s + 1) * ncL / a.nsplit);
  const int max_row = a.num_blocks * a.Hkv * kBlockTokens - 1;

  // QK B operand (Q^T): lane holds column n16, dims kk*32 + q4*8 .. +8.
  bf16x8 qf[KK];
  {
    const uint16_t* qrow =
        a.q + ((size_t)(b * a.T + col_t) * a.Hq + h * a.G + col_g) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (col_valid) v = *reinterpret_cast<const uint4*>(qrow + kk * 32 + q4 * 8);
      qf[kk] = as_bf16x8(v);
    }
  }

  // This lane's key slices: dims kk*32 + q4*8 .. +8 of row r are at
  // kb[kk] + r * kld[kk].
  const uint16_t* kb[KK];
  uint32_t kld[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int dim = kk * 32 + q4 * 8;
    if (!SPLIT) {
      kb[kk] = a.k_cache + dim;
      kld[kk] = D;
    } else {
      const int lo = 2 * a.pair_begin;
      const int nd = 2 * a.pair_count;
      const bool scored = dim >= lo && dim < lo + nd;
      const uint16_t* rest = a.k_rest ? a.k_rest : a.k_cache;  // no rest dims when nd == D
      kb[kk] = scored ? a.k_cache + (dim - lo) : rest + (dim < lo ? dim : dim - nd);
      kld[kk] = scored ? nd : D - nd;
    }
  }

  float m_run = -INFINITY;  // state of head n16 (replicated over q4)
  float l_run = 0.0f;
  f32x4 acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int* btrow = a.block_table + (size_t)b * a.max_blocks;
  const size_t seg = (size_t)u * a.seg_ld;
  // The split's first chunk when the span covers every chunk: its counts and
  // first batch of items are read together with the query, ahead of the
  // sequence length that decides the chunk range (used only if it matches).
  const int c_guess = (int)((int64_t)s * a.nchunk / a.nsplit);
  const int32_t* cnt_guess = a.sel_cnt + ((size_t)u * a.nchunk + c_guess) * 2;
  const int pf_cnt0 = cnt_guess[0], pf_cnt1 = cnt_guess[1];
  int pf_idx[kBatch / 64];
  float pf_lw[kBatch / 64];
#pragma unroll
  for (int k = 0; k < kBatch / 64; ++k) {
    pf_idx[k] = a.sel_idx[seg + (size_t)c_guess * kChunk + lane + 64 * k];
    pf_lw[k] = a.sel_logw[seg + (size_t)c_guess * kChunk + lane + 64 * k];
  }
  for (int c = c_begin; c < c_end; ++c) {
    const bool guessed = c == c_guess;
    const int32_t* cntp = a.sel_cnt + ((size_t)u * a.nchunk + c) * 2;
    // Counts of a caller-provided selection are clamped to the segment and
    // rows to the cache; positions at or past the member's span are masked:
    // no value can address outside the buffers.
    const int cnt = min(max(guessed ? pf_cnt0 : cntp[0], 0) + max(guessed ? pf_cnt1 : cntp[1], 0),
                        kChunk);
    const int i_lo = (int)((int64_t)sub * cnt / a.nsub);  // this wave's share
    const int i_hi = (int)((int64_t)(sub + 1) * cnt / a.nsub);
    const int32_t* idxp = a.sel_idx + seg + (size_t)c * kChunk;
    const float* lwp = a.sel_logw + seg + (size_t)c * kChunk;
    for (int b0 = i_lo; b0 < i_hi; b0 += kBatch) {
      // Resolve up to kBatch items to cache rows (independent loads), into LDS.
      const int nb = min(kBatch, i_hi - b0);
#pragma unroll
      for (int k = 0; k < kBatch / 64; ++k) {
        const int i = lane + 64 * k;
        int row = -1, pos = 0;  // rows given directly carry no position
        float lw = -INFINITY;
        if (i < nb) {
          const bool pre = guessed && b0 == 0;  // items 0 .. kBatch - 1 of the guessed chunk
          const int v = pre ? pf_idx[k] : idxp[b0 + i];
          lw = pre ? pf_lw[k] : lwp[b0 + i];
          if (a.idx_are_rows) {
            row = min(max(v, 0), max_row);
          } else if (v < L) {  // positions past every member's span are dropped
            pos = max(v, 0);
            int blk = btrow[pos >> 4];
            blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
            row = (blk * a.Hkv + h) * kBlockTokens + (pos & 15);
          } else {
            lw = -INFINITY;
          }
        }
        rows_sh[i] = row;
        lw_sh[i] = lw;
        pos_sh[i] = pos;
      }
      if (lane < 32) {
        rows_sh[kBatch + lane] = -1;
        lw_sh[kBatch + lane] = -INFINITY;
        pos_sh[kBatch + lane] = 0;
      }
      __syncthreads();
      for (int t0 = 0; t0 < nb; t0 += 32) {
        // QK for the two 16-token halves: A = K rows (token n16 of the half).
        f32x4 sc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r = rows_sh[t0 + 16 * hh + n16];
          bf16x8 kf[KK];
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (r >= 0) v = *reinterpret_cast<const uint4*>(kb[kk] + (size_t)r * kld[kk]);
            kf[kk] = as_bf16x8(v);
          }
          f32x4 d = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk)
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[kk], d, 0, 0, 0);
          sc[hh] = d;
        }
        // V rows of this lane's 8 k-slots (issued before the softmax math).
        typename VS::T vr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = (i < 4) ? (4 * q4 + i) : (16 + 4 * q4 + (i - 4));
          const int r = rows_sh[t0 + tok];
          vr[i] = VS::zero();
          if (r >= 0)
            vr[i] = *reinterpret_cast<const typename VS::T*>(a.v_cache + (size_t)r * D + n16 * DPL);
        }
        // Logits of (column n16, slot tokens), online softmax update; a
        // column ignores positions past its member's span.
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = (i < 4) ? (4 * q4 + i) : (16 + 4 * q4 + (i - 4));
          x[i] = pos_sh[t0 + tok] < L_col ? sc[i >> 2][i & 3] * a.scale + lw_sh[t0 + tok]
                                          : -INFINITY;
          tmax = fmaxf(tmax, x[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        // A tile of masked entries only (m_new still -inf) must add nothing:
        // exponentiate against 0 instead of -inf.
        const float m_ref = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __expf(m_run - m_ref);
        float psum = 0.0f;
        uint32_t phi[4], plo[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float p0 = __expf(x[i] - m_ref);
          const float p1 = __expf(x[i + 1] - m_ref);
          psum += p0 + p1;
          const uint32_t h0 = f32_to_bf16_bits(p0), h1 = f32_to_bf16_bits(p1);
          const uint32_t l0 = f32_to_bf16_bits(p0 - __uint_as_float(h0 << 16));
          const uint32_t l1 = f32_to_bf16_bits(p1 - __uint_as_float(h1 << 16));
          phi[i >> 1] = h0 | (h1 << 16);
          plo[i >> 1] = l0 | (l1 << 16);
        }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // Rescale the accumulators: rows 4*q4 + r belong to column 4*q4 + r,
        // whose alpha sits in lane 4*q4 + r.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, 4 * q4 + r);
#pragma unroll
          for (int j = 0; j < DPL; ++j) acc[j][r] *= ar;
        }
        const bf16x8 pa_hi = as_bf16x8(make_uint4(phi[0], phi[1], phi[2], phi[3]));
        const bf16x8 pa_lo = as_bf16x8(make_uint4(plo[0], plo[1], plo[2], plo[3]));
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const int w = j >> 1;
          uint32_t p[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t w0 = VS::word(vr[2 * k], w), w1 = VS::word(vr[2 * k + 1], w);
            p[k] = (j & 1) ? pack_hi(w0, w1) : pack_lo(w0, w1);
          }
          const bf16x8 vb = as_bf16x8(make_uint4(p[0], p[1], p[2], p[3]));
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vb, acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb, acc[j], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }

  // Write this split's state: acc rows are query columns 4*q4 + r (member,
  // head); lane column n16 holds dims n16*DPL .. +DPL.
  const int stride = D + 2;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int col = 4 * q4 + r;
    if (col < nmem * a.G) {
      const int qrow = (b * a.T + t_a + col / a.G) * a.Hq + h * a.G + col % a.G;
      float* dst = a.part + ((size_t)qrow * nslot + slot) * stride + n16 * DPL;
#pragma unroll
      for (int j = 0; j < DPL; ++j) dst[j] = acc[j][r];
    }
  }
  if (q4 == 0 && col_valid) {
    const int qrow = (b * a.T + col_t) * a.Hq + h * a.G + col_g;
    float* dst = a.part + ((size_t)qrow * nslot + slot) * stride + D;
    dst[0] = m_run;
    dst[1] = l_run;
  }
}

// Merge of the split states of one (query position, query head), for one
// 64-dim slice of the head (grid: B*T*Hq x d/64):
//   m* = max_s m_s,  o = sum_s e^{m_s - m*} acc_s / sum_s e^{m_s - m*} l_s,
// in a fixed order (deterministic).  The split weights e^{m_s - m*} are
// computed once into LDS; each wave then takes every kMW-th split (lane =
// dim, so one split's slice is one contiguous wave-wide load).
constexpr int kMT = 256;
constexpr int kMW = kMT / 64;
constexpr int kMaxMergeSplits = SSA_MAX_SEQ_LEN / kChunk;

__global__ __launch_bounds__(kMT) void merge_kernel(AttendArgs a) {
  __shared__ float red[kMW];
  __shared__ float esh[kMaxMergeSplits];
  __shared__ float accsh[kMW][64];
  const int bh = blockIdx.x;
  const int D = a.d;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int dim = blockIdx.y * 64 + lane;
  const int ns = a.nsplit * a.nsub;
  const float* base = a.part + (size_t)bh * ns * (D + 2);
  float mx = -INFINITY;
  for (int s = threadIdx.x; s < ns; s += kMT) {
    const float m = base[(size_t)s * (D + 2) + D];
    esh[s] = m;
    mx = fmaxf(mx, m);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float mstar = red[0];
#pragma unroll
  for (int w = 1; w < kMW; ++w) mstar = fmaxf(mstar, red[w]);
  __syncthreads();
  float den = 0.0f;
  for (int s = threadIdx.x; s < ns; s += kMT) {
    const float m = esh[s];
    const float e = (m != -INFINITY) ? __expf(m - mstar) : 0.0f;
    esh[s] = e;
    den += e * base[(size_t)s * (D + 2) + D + 1];
  }
  den = wave_sum(den);
  if (lane == 0) red[wave] = den;
  __syncthreads();
  float denom = 0.0f;
#pragma unroll
  for (int w = 0; w < kMW; ++w) denom += red[w];
  float o = 0.0f;
#pragma unroll 16
  for (int s = wave; s < ns; s += kMW) o += esh[s] * base[(size_t)s * (D + 2) + dim];
  accsh[wave][lane] = o;
  __syncthreads();
  if (threadIdx.x < 64) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kMW; ++w) t += accsh[w][threadIdx.x];
    const float res = (mstar == -INFINITY || denom <= 0.0f) ? 0.0f : t / denom;
    if (a.out_dtype == SSA_BF16)
      reinterpret_cast<uint16_t*>(a.out)[(size_t)bh * D + dim] = (uint16_t)f32_to_bf16_bits(res);
    else
      reinterpret_cast<float*>(a.out)[(size_t)bh * D + dim] = res;
  }
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t stream) {
  dim3 grid(a.nsplit * a.nsub, a.B * a.NG * a.Hkv * a.mblocks);
  // Split keys whose scored dims cover the whole head (no rest array) are
  // addressed exactly like whole keys.
  const bool split = a.k_rest != nullptr;
  if (a.d == 128 && !split)
    attend_kernel<128, false><<<grid, 64, 0, stream>>>(a);
  else if (a.d == 128)
    attend_kernel<128, true><<<grid, 64, 0, stream>>>(a);
  else if (a.d == 64 && !split)
    attend_kernel<64, false><<<grid, 64, 0, stream>>>(a);
  else if (a.d == 64)
    attend_kernel<64, true><<<grid, 64, 0, stream>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge(const AttendArgs& a, hipStream_t stream) {
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  merge_kernel<<<dim3(a.B * a.T * a.Hq, a.d / 64), kMT, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ssa

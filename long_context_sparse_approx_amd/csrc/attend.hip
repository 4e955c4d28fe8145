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
#include "select_device.h"
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

// The tiles of one batch of nb resolved items (rows_sh: cache row or -1,
// lw_sh: logit bias, pos_sh: position for the span mask; entries nb ..
// nb + 31 are padding), folded into the wave's online-softmax state.
template <int D, bool SPLIT>
__device__ __forceinline__ void attend_tiles(const AttendArgs& a, int nb, const int* rows_sh,
                                             const float* lw_sh, const int* pos_sh,
                                             const bf16x8 (&qf)[D / 32],
                                             const uint16_t* const (&kb)[D / 32],
                                             const uint32_t (&kld)[D / 32], int L_col, int n16,
                                             int q4, float& m_run, float& l_run,
                                             f32x4 (&acc)[D / 16]) {
  constexpr int KK = D / 32;
  constexpr int DPL = D / 16;
  using VS = VSlice<D>;
  for (int t0 = 0; t0 < nb; t0 += 32) {
    // QK for the two 16-token halves: A = K rows (token n16 of the half).
    // Every K load of the tile is unconditional (a marked item reads row 0
    // and is zeroed), so the eight loads are in flight together; the V
    // loads follow the same way once the QK products are issued.
    bf16x8 kf[2][KK];
    bool kok[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = rows_sh[t0 + 16 * hh + n16];
      kok[hh] = r >= 0;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kf[hh][kk] =
            as_bf16x8(*reinterpret_cast<const uint4*>(kb[kk] + (size_t)max(r, 0) * kld[kk]));
    }
    f32x4 sc[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (!kok[hh]) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kf[hh][kk] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
      }
      f32x4 d = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[hh][kk], qf[kk], d, 0, 0, 0);
      sc[hh] = d;
    }
    // V rows of this lane's 8 k-slots (issued before the softmax math, and
    // kept after the QK products so that K and V registers are not live
    // together).
    __builtin_amdgcn_sched_barrier(0);
    typename VS::T vr[8];
    bool vok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = (i < 4) ? (4 * q4 + i) : (16 + 4 * q4 + (i - 4));
      const int r = rows_sh[t0 + tok];
      vok[i] = r >= 0;
      vr[i] = *reinterpret_cast<const typename VS::T*>(a.v_cache + (size_t)max(r, 0) * D +
                                                      n16 * DPL);
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
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!vok[i]) vr[i] = VS::zero();
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
}

// SPLIT: the keys are held in two arrays of the same row numbering: the
// scored dims (2 * pair_count per row) apart from the others ("FASA:
// Frequency-aware Sparse Attention", section 3, variants: FASA-M keeps the
// dominant key components resident and moves the rest of the key and the
// values elsewhere); a row is put back together from its 16-byte slices.
template <int D, bool SPLIT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void attend_kernel(
    AttendArgs a) {
  constexpr int KK = D / 32;   // QK steps over the head dim
  constexpr int DPL = D / 16;  // head dims per PV column = PV steps
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
      attend_tiles<D, SPLIT>(a, nb, rows_sh, lw_sh, pos_sh, qf, kb, kld, L_col, n16, q4, m_run,
                             l_run, acc);
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

// ------------------------------------------------------------------ fused
// The decode step (without early stopping or refine) takes the sample
// stage's decisions in the attention wave, per chunk, instead of reading a
// written selection ("Stratified Sparse Attention speeds up decoding 2.96x at 1M
// context", "How SSA stratifies the cache": the deterministic stratum and
// the Poisson-sampled tail with inclusion probability min(1, m w / W)).  The
// decisions and their order are the sample kernel's: tokens above the
// threshold digit and candidates above the threshold key (or within the tie
// quota, ranked by position) are deterministic; the listed tail tokens and
// the other candidates pass fl(u W) < fl(m w) with u from Philox4x32-10 and
// carry the bias -log(min(1, m w / W)); the chunk's items are deterministic
// positions ascending, then sampled positions ascending.  So the output is
// bitwise that of the staged path (selection, then attention over it).
//
// Each wave marks the chunk's decisions in two LDS bitmaps, takes each
// word's rank offset from a wave scan, and places every item at its rank.
// Lists of up to 128 entries (the common case: about 80 selected tokens per
// 4096-token chunk at 50x sparsity) are held in registers, two entries per
// lane, with the sampled entries' biases; longer ones are read in rounds of
// 64 and their biases go through a position-indexed scratch row.  Dense
// units take every valid position.
constexpr int kSelWords = kChunk / 32;
constexpr int kChunkBlocks = kChunk / kBlockTokens;
constexpr int kRegList = 128;  // entries of each list held in registers

struct SelShared {
  uint32_t map[2][kSelWords];  // positions of the chunk: [0] deterministic, [1] sampled
  int blk[kChunkBlocks];       // the chunk's cache block ids (clamped)
};

// A chunk's counts and the first two rounds of its lists (entries past a
// count are read from the segment and never used).
struct ChunkLists {
  int n_above, n_samp, ncand, before, ties_here;
  int lt[2];
  float lwv[2];
  int ct[2];
  uint32_t ck[2];
  float cwv[2];
  int blk[kChunkBlocks / 64];
};

__device__ __forceinline__ ChunkLists load_chunk_lists(const AttendArgs& a, size_t seg,
                                                       size_t ci, int c, int b, int lane) {
  ChunkLists r;
  const size_t base = seg + (size_t)c * kChunk + lane;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    r.lt[k] = a.list_idx[base + 64 * k];
    r.lwv[k] = a.list_w[base + 64 * k];
    r.ct[k] = a.cand_idx[base + 64 * k];
    r.ck[k] = a.cand_key[base + 64 * k];
    r.cwv[k] = a.cand_w[base + 64 * k];
  }
  const int* bt = a.block_table + (size_t)b * a.max_blocks;
#pragma unroll
  for (int k = 0; k < kChunkBlocks / 64; ++k)
    r.blk[k] = bt[min(c * kChunkBlocks + lane + 64 * k, a.max_blocks - 1)];
  r.n_above = a.list_cnt[2 * ci];
  r.n_samp = a.list_cnt[2 * ci + 1];
  r.ncand = a.cand_cnt[ci];
  r.before = a.ties_before[ci];
  r.ties_here = a.tiecnt[ci];
  return r;
}

// The sample stage's inclusion test of tail token t with weight w; *bias
// gets -log(pi) when it passes.
__device__ __forceinline__ bool fused_sample(const UnitState& st, uint64_t seed, int b, int h,
                                             int grp, int t, float w, float* bias) {
  const uint4 wd = philox_block(seed, b, h, (uint32_t)t >> 2, grp);
  const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
  const float mw = (float)st.m * w;
  if (uniform24(words[t & 3]) * st.W < mw) {
    *bias = -logf(fminf(1.0f, mw / st.W));
    return true;
  }
  return false;
}

// The same test without a branch, for slots computed side by side: *bias is
// written whatever the outcome (used only where the test passes).
__device__ __forceinline__ bool sample_test(const UnitState& st, uint64_t seed, int b, int h,
                                            int grp, int t, float w, float* bias) {
  const uint4 wd = philox_block_uniform_key(seed, b, h, (uint32_t)t >> 2, grp);
  const uint32_t word = (t & 2) ? ((t & 1) ? wd.w : wd.z) : ((t & 1) ? wd.y : wd.x);
  const float mw = (float)st.m * w;
  *bias = -logf(fminf(1.0f, mw / st.W));
  return uniform24(word) * st.W < mw;
}

__device__ __forceinline__ void mark(uint32_t* map, int p) {
  atomicOr(&map[p >> 5], 1u << (p & 31));
}

// MULTI: several query positions per sequence (member blocks on grid z, each
// column its own causal span, entries placed with their positions); without
// it, one query per sequence (grid y = unit = b * Hkv + h, rows only).
template <int D, bool SPLIT, bool MULTI>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void attend_select_kernel(
    AttendArgs a) {
  constexpr int KK = D / 32;
  constexpr int DPL = D / 16;
  __shared__ int rows_sh[kBatch + 32];
  __shared__ float lw_sh[kBatch + 32];
  __shared__ int pos_sh[kBatch + 32];
  __shared__ SelShared ssh;

  const int slot = blockIdx.x;
  const int s = slot / a.nsub;
  const int sub = slot - s * a.nsub;
  const int nslot = a.nsplit * a.nsub;
  const int u = blockIdx.y;
  const int bg = u / a.Hkv;
  const int h = u - bg * a.Hkv;
  int b = bg, grp = 0, t_a = 0, nmem = 1;
  if (MULTI) {
    b = bg / a.NG;
    grp = bg - b * a.NG;
    t_a = grp * a.g + (int)blockIdx.z * a.mpw;  // first member of this block
    nmem = min(min(a.mpw, (grp + 1) * a.g - t_a), a.T - t_a);
    if (nmem <= 0) return;  // uniform over the wave
  }
  const int lane = threadIdx.x;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const uint64_t ltmask = (1ull << lane) - 1ull;
  const size_t seg = (size_t)u * a.seg_ld;
  // The split's first chunk when the sequence covers every chunk: its counts,
  // lists and block ids are read with the unit state and the query, ahead of
  // the sequence length that decides the range (used only if it matches).
  // Index arithmetic in 32 bits: s * chunks < 4096 * 4096.
  const int c_guess = (int)((uint32_t)s * (uint32_t)a.nchunk / (uint32_t)a.nsplit);
  const ChunkLists pf = load_chunk_lists(a, seg, (size_t)u * a.nchunk + c_guess, c_guess, b, lane);
  const UnitState st = reinterpret_cast<const UnitState*>(a.state)[u];
  const uint64_t seed = a.seed[b];
  // Column n16 = (member t_a + n16 / G, head n16 % G).
  const bool col_valid = n16 < nmem * a.G;
  const int col_t = MULTI ? t_a + (col_valid ? n16 / a.G : 0) : 0;
  const int col_g = col_valid ? (MULTI ? n16 - (n16 / a.G) * a.G : n16) : 0;
  bf16x8 qf[KK];
  {
    // Loaded for every column, with no branch: a column past the block reads
    // its first member's head 0, and its span is empty (L_col = 0), so its
    // logits are -inf, its probabilities 0 and its state is never written; an
    // MFMA output column depends on its own query column only.
    const uint16_t* qrow = a.q + ((size_t)(b * a.T + col_t) * a.Hq + h * a.G + col_g) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + kk * 32 + q4 * 8));
  }
  // The loads above stay here (a scheduling barrier), in flight while the
  // sequence length and the chunk range are worked out, instead of sinking
  // into the branch that uses them.
  __builtin_amdgcn_sched_barrier(0);
  const int P = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int L_col = col_valid ? (MULTI ? member_span(P, a.T, col_t) : P) : 0;
  const int L = MULTI ? member_span(P, a.T, t_a + nmem - 1) : P;  // the block's widest span
  const int ncL = (L + kChunk - 1) / kChunk;
  const int c_begin = (int)((uint32_t)s * (uint32_t)ncL / (uint32_t)a.nsplit);
  const int c_end = (int)((uint32_t)(s + 1) * (uint32_t)ncL / (uint32_t)a.nsplit);

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
      const uint16_t* rest = a.k_rest ? a.k_rest : a.k_cache;
      kb[kk] = scored ? a.k_cache + (dim - lo) : rest + (dim < lo ? dim : dim - nd);
      kld[kk] = scored ? nd : D - nd;
    }
  }

  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x4 acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const bool empty = (st.flags & kFlagEmpty) != 0;
  const bool dense = (st.flags & kFlagDense) != 0;
  const bool sampling = (st.flags & kFlagSample) != 0;
  const bool use_topk = !(st.flags & kFlagNoTopk);
  // One chunk of the split; false once the unit's span has ended.
  auto do_chunk = [&](int c, const ChunkLists& cl) -> bool {
    const int c0 = c * kChunk;
    if (empty || c0 >= st.L) return false;  // uniform
    const int nvalid = min(kChunk, st.L - c0);
    const int n_above = clamp_count(cl.n_above, kChunk);
    const int n_samp = clamp_count(cl.n_samp, kChunk - n_above);
    const int n_list = n_above + (sampling ? n_samp : 0);
    const int ncand = use_topk ? clamp_count(cl.ncand, kChunk) : 0;
#pragma unroll
    for (int k = 0; k < kChunkBlocks / 64; ++k) {
      const int v = cl.blk[k];
      ssh.blk[lane + 64 * k] = v < 0 ? 0 : (v >= a.num_blocks ? a.num_blocks - 1 : v);
    }
    // mode 0: dense (every valid position, in order); 1: lists in registers;
    // 2: lists read in rounds.
    const int mode = dense ? 0 : (n_list <= kRegList && ncand <= kRegList ? 1 : 2);
    int kd[4] = {0, 0, 0, 0};  // 0 none, 1 deterministic, 2 sampled
    int ps[4] = {0, 0, 0, 0};  // position in the chunk, then rank
    int pp[4] = {0, 0, 0, 0};  // position in the chunk
    int rw[4] = {0, 0, 0, 0};  // cache row
    float bs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int totS = nvalid, totR = 0, ex = 0;
    ssh.map[0][lane] = 0u;
    ssh.map[0][lane + 64] = 0u;
    ssh.map[1][lane] = 0u;
    ssh.map[1][lane + 64] = 0u;
    __syncthreads();
    if (mode != 0) {
      if (mode == 1) {
        // Slots 0, 1: list entries lane, lane + 64; slots 2, 3: candidates.
        // Every slot's inclusion test is computed (four independent Philox
        // blocks side by side) and used where the slot is a tail token.
        const int tt[4] = {cl.lt[0], cl.lt[1], cl.ct[0], cl.ct[1]};
        const float wv[4] = {cl.lwv[0], cl.lwv[1], cl.cwv[0], cl.cwv[1]};
        // A slot none of whose entries is a tail token skips the test (a
        // condition uniform over the wave).
        const bool need[4] = {n_list > n_above, n_list > max(n_above, 64),
                              sampling && ncand > 0, sampling && ncand > 64};
        bool pass[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ps[k] = tt[k] - c0;
          pass[k] = need[k] ? sample_test(st, seed, b, h, grp, tt[k], wv[k], &bs[k]) : false;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int i = lane + 64 * k;
          const bool valid = (unsigned)ps[k] < (unsigned)nvalid;
          if (i < n_above)
            kd[k] = valid ? 1 : 0;
          else if (i < n_list && valid && pass[k])
            kd[k] = 2;
        }
        bool tie[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) tie[k] = lane + 64 * k < ncand && cl.ck[k] == st.tkey;
        const uint64_t tb0 = __ballot(tie[0]);
        const uint64_t tb1 = __ballot(tie[1]);
        const int pre[2] = {(int)__popcll(tb0 & ltmask),
                            (int)(__popcll(tb0) + __popcll(tb1 & ltmask))};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int i = lane + 64 * k;
          const bool valid = (unsigned)ps[2 + k] < (unsigned)nvalid;
          if (i < ncand) {
            const int rank = cl.ties_here != 0 ? cl.before + pre[k] : 0;
            if (cl.ck[k] > st.tkey || (tie[k] && rank < st.ties_needed))
              kd[2 + k] = valid ? 1 : 0;
            else if (sampling && valid && pass[2 + k])
              kd[2 + k] = 2;
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          pp[k] = ps[k];
          if (kd[k] != 0) mark(ssh.map[kd[k] - 1], ps[k]);
          // The cache row, read before the ranks are known.
          rw[k] = (ssh.blk[(ps[k] >> 4) & (kChunkBlocks - 1)] * a.Hkv + h) * kBlockTokens +
                  (ps[k] & 15);
        }
      } else {
        float* scr = a.sel_scratch + seg + (size_t)c * kChunk;
        const int32_t* lidx = a.list_idx + seg + (size_t)c * kChunk;
        const float* lw = a.list_w + seg + (size_t)c * kChunk;
        for (int i = lane; i < n_list; i += 64) {
          const int t = lidx[i];
          const int p = t - c0;
          if ((unsigned)p >= (unsigned)nvalid) continue;
          float bias;
          if (i < n_above)
            mark(ssh.map[0], p);
          else if (fused_sample(st, seed, b, h, grp, t, lw[i], &bias)) {
            scr[p] = bias;
            mark(ssh.map[1], p);
          }
        }
        const int32_t* cidx = a.cand_idx + seg + (size_t)c * kChunk;
        const uint32_t* ckey = a.cand_key + seg + (size_t)c * kChunk;
        const float* cw = a.cand_w + seg + (size_t)c * kChunk;
        int run = 0;
        for (int base = 0; base < ncand; base += 64) {
          const int i = base + lane;
          const bool v = i < ncand;
          const uint32_t key = v ? ckey[i] : 0u;
          const int t = v ? cidx[i] : 0;
          const bool tie = v && key == st.tkey;
          const uint64_t tb = __ballot(tie);
          const int rank = cl.ties_here != 0 ? cl.before + run + __popcll(tb & ltmask) : 0;
          run += __popcll(tb);
          const int p = t - c0;
          if (v && (unsigned)p < (unsigned)nvalid) {
            float bias;
            if (key > st.tkey || (tie && rank < st.ties_needed))
              mark(ssh.map[0], p);
            else if (sampling && fused_sample(st, seed, b, h, grp, t, cw[i], &bias)) {
              scr[p] = bias;
              mark(ssh.map[1], p);
            }
          }
        }
        __threadfence_block();  // the biases, read back by other lanes below
      }
      __syncthreads();
      // Each word's rank offsets: lane l takes words 2l and 2l + 1 (positions
      // 64 l .. 64 l + 63).
      const uint32_t d0 = ssh.map[0][2 * lane], d1 = ssh.map[0][2 * lane + 1];
      const uint32_t s0 = ssh.map[1][2 * lane] & ~d0, s1 = ssh.map[1][2 * lane + 1] & ~d1;
      const int packed = (__popc(d0) + __popc(d1)) | ((__popc(s0) + __popc(s1)) << 16);
      const int inc = wave_inclusive_scan<int>(packed);
      const int tot = __builtin_amdgcn_readlane(inc, 63);
      totS = tot & 0xffff;
      totR = tot >> 16;
      ex = inc - packed;
      if (mode == 1) {
        // Items to ranks, from the owning lane's offsets and words (a sampled
        // item that is also deterministic is dropped, as in the sample
        // kernel; the lists never make one).  Every lane reads go out before
        // any rank is formed.
        int o_ex[4];
        uint32_t o_d0[4], o_d1[4], o_s0[4], o_s1[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int addr = ((ps[k] & (kChunk - 1)) >> 6) << 2;  // owning lane, in bytes
          o_ex[k] = __builtin_amdgcn_ds_bpermute(addr, ex);
          o_d0[k] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)d0);
          o_d1[k] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)d1);
          o_s0[k] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)s0);
          o_s1[k] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)s1);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int bit = ps[k] & 63;
          const uint64_t below = bit == 0 ? 0ull : (~0ull >> (64 - bit));
          const uint64_t dw = ((uint64_t)o_d1[k] << 32) | o_d0[k];
          const uint64_t sw = ((uint64_t)o_s1[k] << 32) | o_s0[k];
          const int rd = (o_ex[k] & 0xffff) + (int)__popcll(dw & below);
          const int rs = totS + (o_ex[k] >> 16) + (int)__popcll(sw & below);
          const bool drop = kd[k] == 2 && ((dw >> bit) & 1ull);
          ps[k] = kd[k] == 1 ? rd : rs;
          bs[k] = kd[k] == 1 ? 0.0f : bs[k];
          kd[k] = drop ? 0 : kd[k];
        }
      }
    }
    // An entry at or past the block's widest span takes its slot with no row
    // (the staged attention drops it the same way); the others carry their
    // position for the members' span masks.
    auto place = [&](int j, int p, int row, float lw) {
      if (MULTI) {
        const int pos = c0 + p;
        const bool in = pos < L;
        rows_sh[j] = in ? row : -1;
        lw_sh[j] = in ? lw : -INFINITY;
        pos_sh[j] = in ? pos : 0;
      } else {  // every entry lies inside the one query's span
        rows_sh[j] = row;
        lw_sh[j] = lw;
        pos_sh[j] = 0;
      }
    };
    const int cnt = totS + totR;
    const int i_lo = (int)((uint32_t)sub * (uint32_t)cnt / (uint32_t)a.nsub);
    const int i_hi = (int)((uint32_t)(sub + 1) * (uint32_t)cnt / (uint32_t)a.nsub);
    if (mode == 1) {
      // At most 2 * kRegList = kBatch items: one batch, placed here so that
      // the items' registers are free during the tiles.
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = ps[k] - i_lo;
        if (kd[k] != 0 && (unsigned)j < (unsigned)(i_hi - i_lo)) place(j, pp[k], rw[k], bs[k]);
      }
    }
    static_assert(2 * kRegList <= kBatch, "the register-held lists fill one batch");
    for (int b0 = i_lo; b0 < i_hi; b0 += kBatch) {
      const int nb = min(kBatch, i_hi - b0);
      if (mode == 0) {
#pragma unroll
        for (int k = 0; k < kBatch / 64; ++k) {
          const int i = lane + 64 * k;
          if (i < nb) {
            const int p = b0 + i;
            place(i, p, (ssh.blk[p >> 4] * a.Hkv + h) * kBlockTokens + (p & 15), 0.0f);
          }
        }
      }
      // Padding: a tile reads at most 31 entries past the batch's last item.
      if (lane < 32) {
        rows_sh[nb + lane] = -1;
        lw_sh[nb + lane] = -INFINITY;
        pos_sh[nb + lane] = 0;
      }
      if (mode == 2) {
        // Lane l's positions 64 l .. 64 l + 63, deterministic then sampled.
        const float* scr = a.sel_scratch + seg + (size_t)c * kChunk;
#pragma unroll
        for (int cls = 0; cls < 2; ++cls) {
          int r = cls == 0 ? (ex & 0xffff) : totS + (ex >> 16);
#pragma unroll
          for (int wj = 0; wj < 2; ++wj) {
            const uint32_t dm = ssh.map[0][2 * lane + wj];
            uint32_t bits = cls == 0 ? dm : ssh.map[1][2 * lane + wj] & ~dm;
            for (; bits != 0u; bits &= bits - 1u, ++r) {
              const int j = r - b0;
              if ((unsigned)j >= (unsigned)nb) continue;
              const int p = 64 * lane + 32 * wj + __builtin_ctz(bits);
              place(j, p, (ssh.blk[p >> 4] * a.Hkv + h) * kBlockTokens + (p & 15),
                    cls == 0 ? 0.0f : scr[p]);
            }
          }
        }
      }
      __syncthreads();
      attend_tiles<D, SPLIT>(a, nb, rows_sh, lw_sh, pos_sh, qf, kb, kld, L_col, n16, q4, m_run,
                             l_run, acc);
      __syncthreads();
    }
    return true;
  };
  // The first chunk takes the prefetched lists when the range starts at the
  // guessed chunk (peeled, so that they are not live across later chunks).
  if (c_begin < c_end) {
    bool go = do_chunk(c_begin, c_begin == c_guess
                                    ? pf
                                    : load_chunk_lists(a, seg, (size_t)u * a.nchunk + c_begin,
                                                       c_begin, b, lane));
    for (int c = c_begin + 1; go && c < c_end; ++c)
      go = do_chunk(c, load_chunk_lists(a, seg, (size_t)u * a.nchunk + c, c, b, lane));
  }

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
// 16-dim slice of the head (grid: B*T*Hq x d/16):
//   m* = max_s m_s,  o = sum_s e^{m_s - m*} acc_s / sum_s e^{m_s - m*} l_s,
// in a fixed order (deterministic).  Thread t takes dim t % 16 of the slice
// for splits t / 16, t / 16 + 16, ...; the first kMSlots of its accumulator
// values go out with the split maxima and sums, so the common merge (at most
// 256 splits) is one round of loads and three barriers, and a head's slices
// are read by d/16 workgroups side by side.  The split weights e^{m_s - m*}
// are computed once into LDS.
constexpr int kMT = 256;
constexpr int kMW = kMT / 64;
constexpr int kMSlice = 16;                // dims per workgroup
constexpr int kMGroups = kMT / kMSlice;    // split groups per workgroup
constexpr int kMSlots = 16;                // accumulator values per thread in the first loads
constexpr int kMaxMergeSplits = SSA_MAX_SEQ_LEN / kChunk;

__global__ __launch_bounds__(kMT) void merge_kernel(AttendArgs a) {
  __shared__ float red_m[kMW];
  __shared__ float red_d[kMW];
  __shared__ float esh[kMaxMergeSplits];
  __shared__ float osh[kMGroups][kMSlice];
  const int bh = blockIdx.x;
  const int D = a.d;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = threadIdx.x / kMSlice;
  const int sub = threadIdx.x % kMSlice;
  const int dim = blockIdx.y * kMSlice + sub;
  const int ns = a.nsplit * a.nsub;
  const size_t stride = (size_t)D + 2;
  const float* base = a.part + (size_t)bh * ns * stride;
  // Every load from a split clamped into range; values of splits past ns are
  // never used.
  const size_t s0 = (size_t)min((int)threadIdx.x, ns - 1);
  const float m0 = base[s0 * stride + D];
  const float l0 = base[s0 * stride + D + 1];
  float av[kMSlots];
#pragma unroll
  for (int i = 0; i < kMSlots; ++i)
    av[i] = base[(size_t)min(grp + kMGroups * i, ns - 1) * stride + dim];
  float mx = (int)threadIdx.x < ns ? m0 : -INFINITY;
  for (int s = threadIdx.x + kMT; s < ns; s += kMT) mx = fmaxf(mx, base[(size_t)s * stride + D]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  float mstar = red_m[0];
#pragma unroll
  for (int w = 1; w < kMW; ++w) mstar = fmaxf(mstar, red_m[w]);
  float den = 0.0f;
  for (int s = threadIdx.x; s < ns; s += kMT) {
    const bool first = s == (int)threadIdx.x;
    const float m = first ? m0 : base[(size_t)s * stride + D];
    const float l = first ? l0 : base[(size_t)s * stride + D + 1];
    const float e = (m != -INFINITY) ? __expf(m - mstar) : 0.0f;
    esh[s] = e;
    den += e * l;
  }
  den = wave_sum(den);
  if (lane == 0) red_d[wave] = den;
  __syncthreads();
  float denom = 0.0f;
#pragma unroll
  for (int w = 0; w < kMW; ++w) denom += red_d[w];
  float o = 0.0f;
#pragma unroll
  for (int i = 0; i < kMSlots; ++i) {
    const int s = grp + kMGroups * i;
    if (s < ns) o += esh[s] * av[i];
  }
  for (int s = grp + kMGroups * kMSlots; s < ns; s += kMGroups)
    o += esh[s] * base[(size_t)s * stride + dim];
  osh[grp][sub] = o;
  __syncthreads();
  if (threadIdx.x < kMSlice) {
    float t = 0.0f;
#pragma unroll
    for (int g = 0; g < kMGroups; ++g) t += osh[g][threadIdx.x];
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

hipError_t launch_attend_select(const AttendArgs& a, hipStream_t stream) {
  if (!a.fused_select) return hipErrorInvalidValue;
  dim3 grid(a.nsplit * a.nsub, a.B * a.NG * a.Hkv, a.mblocks);
  const bool split = a.k_rest != nullptr;
  const bool multi = a.T > 1;
#define SSA_SEL(d, s, m) attend_select_kernel<d, s, m><<<grid, 64, 0, stream>>>(a)
  if (a.d == 128 && !split)
    multi ? SSA_SEL(128, false, true) : SSA_SEL(128, false, false);
  else if (a.d == 128)
    multi ? SSA_SEL(128, true, true) : SSA_SEL(128, true, false);
  else if (a.d == 64 && !split)
    multi ? SSA_SEL(64, false, true) : SSA_SEL(64, false, false);
  else if (a.d == 64)
    multi ? SSA_SEL(64, true, true) : SSA_SEL(64, true, false);
  else
    return hipErrorInvalidValue;
#undef SSA_SEL
  return hipGetLastError();
}

hipError_t launch_merge(const AttendArgs& a, hipStream_t stream) {
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  merge_kernel<<<dim3(a.B * a.T * a.Hq, a.d / kMSlice), kMT, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ssa

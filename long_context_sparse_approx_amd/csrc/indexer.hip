// Stage 1: approximate scores of every cached token.
//
// "FASA: Frequency-aware Sparse Attention", section 3 stage 1 (TIP): the
// online score of a token sums the contributions of a fixed subset of RoPE
// frequency chunks only.  The group's queries are averaged into one proxy
// query ("PIVOT slashes sparse-attention indexer cost", "The two observations
// behind PIVOT"), so a kv head streams its keys once for its whole query group.
//
// Memory shape.  The scored pairs are a contiguous dim range, so each token
// contributes one contiguous 2*pair_count*2-byte slice of its key row (128 B
// for 32 pairs at d = 128).  LPT lanes cover one token with one 16-byte
// streaming load each; a wave instruction therefore reads 64/LPT token slices
// and every lane keeps 8 independent loads (8 consecutive tokens) in flight.
// The scaled proxy query lives in registers as three bf16 parts (hi + mid +
// lo, float32 precision) and the slices are dotted with v_dot2_f32_bf16
// straight from the loaded words.  A DPP reduce-scatter
// across the LPT lanes leaves each lane with complete token scores, so the
// score stores are coalesced.  The epilogue counts each score's first radix
// digit (top 11 bits of the order key) in an LDS histogram and tracks the
// maximum order key; both are flushed with integer atomics, so the result is
// independent of scheduling.
//
// Work split.  The grid is the number of workgroups the device holds at once,
// and the units' tokens, laid end to end, are split evenly among them (below),
// so the whole layer streams in one round whatever the mix of sequence
// lengths.
#include <atomic>

#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

namespace {

// Largest token tile of one indexer workgroup (its block ids and its scores
// are staged in LDS: 8192 tokens keep four workgroups per CU resident, and
// the tile's scores are written in one burst at its end).  A 1M-token,
// 8-head layer gives each of the 1024 resident workgroups one full tile.
constexpr int kMaxTileTokens = 8192;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load that does not keep the line in the caches (the key
// slices are read once per step).
// Raw (untyped) buffer resources: the fourth descriptor word for 32-bit
// data on this family, and the cache-policy bits of a buffer access (sc0 = 1,
// nt = 2, sc1 = 16).
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kPolicySystem = 1 | 16;

__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float dot2(uint32_t k2, uint32_t q2, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k2),
                                         __builtin_bit_cast(bf16x2, q2), acc, false);
}

// Partial score of one 8-dim key slice: the proxy query is held as three
// bf16 parts (hi + mid + lo: 24 significant bits, float32's precision);
// bf16 x bf16 products are exact and accumulate in fp32.  The key words are
// already in registers, so the third part costs VALU only (the kernel is
// bound by HBM).
__device__ __forceinline__ float slice_dot(const uint32_t* qh, const uint32_t* qm,
                                           const uint32_t* ql, u32x4 k) {
  float s = dot2(k.x, qh[0], 0.0f);
  s = dot2(k.y, qh[1], s);
  s = dot2(k.z, qh[2], s);
  s = dot2(k.w, qh[3], s);
  s = dot2(k.x, qm[0], s);
  s = dot2(k.y, qm[1], s);
  s = dot2(k.z, qm[2], s);
  s = dot2(k.w, qm[3], s);
  s = dot2(k.x, ql[0], s);
  s = dot2(k.y, ql[1], s);
  s = dot2(k.z, ql[2], s);
  s = dot2(k.w, ql[3], s);
  return s;
}

// Value of the partner lane across lane-index bit `bit` (bits 0-2 within
// 8-lane groups, bit 3 within 16-lane rows), through DPP.
template <int BIT>
__device__ __forceinline__ float partner(float x) {
  constexpr int ctrl = BIT == 0 ? 0xB1 : (BIT == 1 ? 0x4E : (BIT == 2 ? 0x141 : 0x128));
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl,
                                                               0xf, 0xf, false));
}

// One reduce-scatter step across lane bit BIT on the first 2*H values: the
// lane whose bit is 0 keeps the first H sums, its partner the last H.
template <int BIT, int H>
__device__ __forceinline__ void rs_step(float* v, bool upper) {
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float keep = upper ? v[H + i] : v[i];
    const float send = upper ? v[i] : v[H + i];
    v[i] = keep + partner<BIT>(send);
  }
}

// LPT lanes cover one token's slice (LPT in 1..16, a power of two); each lane
// holds partial sums of UNR = 8 tokens r.  After the reduce-scatter lane
// position p (= lane % LPT, taken mod 8) holds the complete sums of
// r = p * E + e, e < E, with E = 8 / min(LPT, 8).
template <int LPT>
__device__ __forceinline__ void reduce_scatter(float* v, int lane) {
  if constexpr (LPT == 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += partner<3>(v[i]);
  }
  if constexpr (LPT >= 8) rs_step<2, 4>(v, (lane >> 2) & 1);
  if constexpr (LPT >= 4) rs_step<1, (LPT >= 8 ? 2 : 4)>(v, (lane >> 1) & 1);
  if constexpr (LPT >= 2) rs_step<0, (LPT >= 8 ? 1 : (LPT == 4 ? 2 : 4))>(v, lane & 1);
}

// One wave iteration over TPI * UNR consecutive tokens: lane group g (of LPT
// lanes) takes tokens base + 8 g .. base + 8 g + 7, one 16-byte slice of each
// per lane, all inside one cache block.  After the reduce-scatter, lane
// position p of group g holds the complete scores of tokens
// base + 8 g + p * E + e (e < E), so for LPT = 8 lane l holds token base + l
// and the score stores are contiguous.  FULL: every token is below t_end (no
// predication; all loads are issued back to back).  Scores go to the
// workgroup's LDS tile buffer; the tile is written to HBM in one burst at the
// end (interleaving small score writes with the key stream costs far more HBM
// time than the 4 bytes per token suggest).  The first-digit histogram holds
// two 16-bit counts per word (a tile has at most 8192 tokens).
template <int LPT, bool FULL>
__device__ __forceinline__ void index_iteration(const uint16_t* kbase, const uint32_t* blk_sh,
                                                uint64_t blk_stride, int d, int t0, int base,
                                                int t_end,
                                                const uint32_t* qh, const uint32_t* qm,
                                                const uint32_t* ql, float* sbuf, uint32_t* hist,
                                                uint32_t& kmax,
                                                int lane) {
  constexpr int UNR = 8;
  constexpr int LG = LPT < 8 ? LPT : 8;
  constexpr int E = UNR / LG;
  const int grp = lane / LPT;
  const int pos = (lane % LPT) % LG;
  const bool writer = LPT <= 8 || (lane & 8) == 0;
  const int tg = base + UNR * grp;  // first token of this lane's group (a multiple of 8)
  // A group past the tile's end (ragged iteration only) loads nothing; it
  // takes block 0's id so that its LDS read stays inside the tile's ids.
  const int bi = (FULL || tg < t_end) ? (tg - t0) >> 4 : 0;
  const uint16_t* row0 =
      kbase + (uint64_t)blk_sh[bi] * blk_stride + (uint64_t)(tg & 15) * d;
  u32x4 kv[UNR];
#pragma unroll
  for (int r = 0; r < UNR; ++r)
    kv[r] = (FULL || tg + r < t_end) ? load_stream(row0 + (size_t)r * d) : u32x4{0u, 0u, 0u, 0u};
  float v[UNR];
#pragma unroll
  for (int r = 0; r < UNR; ++r) v[r] = slice_dot(qh, qm, ql, kv[r]);
  reduce_scatter<LPT>(v, lane);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int t = tg + pos * E + e;
    if (writer && (FULL || t < t_end)) {
      sbuf[t - t0] = v[e];
      const uint32_t key = order_key(v[e]);
      const uint32_t bin = key >> kDigit1Shift;
      atomicAdd(&hist[bin >> 1], 1u << (16 * (bin & 1u)));
      kmax = key > kmax ? key : kmax;
    }
  }
}

// One tile [t0, t_end) of unit u (at most kMaxTileTokens tokens, t0 a
// multiple of 16): proxy query, block ids, the key stream, then the tile's
// histogram, maximum and scores.  Called by all threads of the workgroup.
template <int LPT>
__device__ __forceinline__ void index_tile(const IndexArgs& a, int u, int t0, int t_end,
                                           uint32_t* hist, uint32_t* blk_sh, float* sbuf,
                                           uint32_t* wmax) {
  constexpr int TPI = kWave / LPT;           // tokens per wave-wide load
  constexpr int UNR = 8;                     // loads in flight per lane
  constexpr int WAVE_TOK = TPI * UNR;        // tokens per wave per iteration
  constexpr int WG_TOK = 4 * WAVE_TOK;       // tokens per workgroup per iteration
  // The query group's scored slice (at most 16 x 128 floats) is staged in the
  // score tile buffer before the first score lands there.
  static_assert(16 * 128 <= kMaxTileTokens, "query slice fits the tile buffer");
  float* qsh = sbuf;

  const UnitInfo ui = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len);
  const int b = ui.b;
  const int h = ui.h;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nd = 2 * a.pair_count;
  const int sub = lane % LPT;
  // The tile's block ids (their loads go out with the query's).
  const int blk0 = t0 / kBlockTokens;
  const int nblk = (t_end - t0 + kBlockTokens - 1) / kBlockTokens;
  const int* btrow = a.block_table + (size_t)b * a.max_blocks;
  const uint64_t blk_stride = (uint64_t)a.Hkv * kBlockTokens * a.key_ld;
  for (int i = tid; i < nblk; i += 256) {
    const int blk = btrow[blk0 + i];
    blk_sh[i] = (uint32_t)(blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk));
  }
  // Proxy query: the mean over the group's members (consecutive query
  // positions) and their G query heads, accumulated member by member.
  const int t_first = ui.grp * a.g;
  const int t_last = min(t_first + a.g, a.T);
  float qf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qf[i] = 0.0f;
  for (int t = t_first; t < t_last; ++t) {
    for (int i = tid; i < a.G * nd; i += 256) {
      const int g = i / nd;
      const int e = i - g * nd;
      const uint16_t bits =
          a.q[((size_t)(b * a.T + t) * a.Hq + h * a.G + g) * a.d + 2 * a.pair_begin + e];
      qsh[i] = __uint_as_float((uint32_t)bits << 16);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = 0.0f;
      for (int g = 0; g < a.G; ++g) s += qsh[g * nd + sub * 8 + i];
      qf[i] += s;
    }
    __syncthreads();
  }
  // Per-lane proxy query over this lane's 8 dims, qbar = (scale / (G n)) *
  // sum over the n members and G heads, split into bf16 hi, mid and lo parts
  // (each the rounding of what the previous parts leave) packed two dims per
  // word.
  uint32_t qh[4], qm[4], ql[4];
  {
    const float qscale = a.scale / (float)(a.G * (t_last - t_first));
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[i] *= qscale;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t part[3][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float r = qf[2 * i + j];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          part[k][j] = f32_to_bf16_bits(r);
          r -= __uint_as_float(part[k][j] << 16);
        }
      }
      qh[i] = part[0][0] | (part[0][1] << 16);
      qm[i] = part[1][0] | (part[1][1] << 16);
      ql[i] = part[2][0] | (part[2][1] << 16);
    }
  }
  for (int i = tid; i < kBins / 2; i += 256) hist[i] = 0u;
  __syncthreads();

  const uint16_t* kbase = a.k_cache + (size_t)h * kBlockTokens * a.key_ld + a.key_off + sub * 8;
  float* srow = a.scores + (size_t)u * a.score_ld;
  uint32_t kmax = 0u;
  // A CU serves its oldest waves first, so workgroups that share a CU would
  // stream at very different rates and the late ones would finish alone with
  // few loads in flight.  Each wave therefore lowers its priority as it
  // advances (3 up to 60% of its tile, then 2, 1 from 85%, 0 from 95%): a
  // wave that is ahead yields to those behind, and the CU's workgroups finish
  // together.  The bands narrow towards the end, where the spread matters.
  int base = t0 + wave * WAVE_TOK;
  const int n_full = base + WAVE_TOK <= t_end ? (t_end - WAVE_TOK - base) / WG_TOK + 1 : 0;
  __builtin_amdgcn_s_setprio(3);
  int level = 0;  // priority bands passed
  for (int it = 0; it < n_full; ++it, base += WG_TOK) {
    const int q = (it * 20 >= 12 * n_full) + (it * 20 >= 17 * n_full) + (it * 20 >= 19 * n_full);
    if (q != level) {
      level = q;
      if (q == 1)
        __builtin_amdgcn_s_setprio(2);
      else if (q == 2)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
    index_iteration<LPT, true>(kbase, blk_sh, blk_stride, a.key_ld, t0, base, t_end, qh, qm, ql,
                               sbuf, hist, kmax, lane);
  }
  __builtin_amdgcn_s_setprio(0);
  if (base < t_end)
    index_iteration<LPT, false>(kbase, blk_sh, blk_stride, a.key_ld, t0, base, t_end, qh, qm, ql,
                                sbuf, hist, kmax, lane);

  kmax = wave_max_u32(kmax);
  if (lane == 0) wmax[wave] = kmax;
  __syncthreads();
  if (tid == 0) {
    uint32_t mx = wmax[0];
    for (int w = 1; w < 4; ++w) mx = wmax[w] > mx ? wmax[w] : mx;
    atomicMax(&a.maxkey[u], mx);
  }
  for (int i = tid; i < kBins; i += 256) {
    const uint32_t c = (hist[i >> 1] >> (16 * (i & 1))) & 0xffffu;
    if (c) atomicAdd(&a.hist1[(size_t)u * kBins + i], c);
  }
  // The tile's scores, written in one burst (16-byte stores when aligned)
  // with the system-scope cache policy (sc0 sc1): written through instead of
  // left dirty in L2 for the key stream to evict piecemeal, which costs the
  // stream less HBM time (1M layer: 173 -> 169 us).  The buffer resource
  // spans the unit's score row, so every store is range-checked against it.
  const int n = t_end - t0;
  float* dst = srow + t0;
  if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
    const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
        srow, (short)0, (int)(uint32_t)(a.score_ld * (int64_t)sizeof(float)), kRawBufferWord3);
    for (int i = 4 * tid; i < n; i += 4 * 256) {
      if (i + 4 <= n) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(sbuf + i);
        __builtin_amdgcn_raw_buffer_store_b128(v, row, (uint32_t)(t0 + i) * 4u, 0, kPolicySystem);
      } else {
        for (int j = i; j < n; ++j) dst[j] = sbuf[j];
      }
    }
  } else {
    for (int i = tid; i < n; i += 256) dst[i] = sbuf[i];
  }
  __syncthreads();  // the tile buffer and histogram are reused by the next tile
}

// Work split.  Every unit's token range, rounded up to kFlatAlign tokens, is
// laid end to end in unit order; workgroup w takes the w-th of gridDim.x
// equal shares of that space (whole multiples of kFlatAlign), so any mix of
// sequence lengths keeps the workgroups equally busy, and equal lengths give
// each workgroup one contiguous tile.  A share is processed as tiles of at
// most kMaxTileTokens tokens of one unit; padding past a unit's length is
// skipped.  Every workgroup derives the split from seq_lens itself.
constexpr int kFlatAlign = kIndexAlign;

__device__ __forceinline__ int unit_len(const IndexArgs& a, int u) {
  return unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len).L;
}

__device__ __forceinline__ unsigned long long padded(int L) {
  return (unsigned long long)((L + kFlatAlign - 1) / kFlatAlign) * kFlatAlign;
}

__device__ __forceinline__ unsigned long long padded_len(const IndexArgs& a, int u) {
  return u < a.units ? padded(unit_len(a, u)) : 0ull;
}

// A value the whole wave holds, moved to scalar registers.
__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Both halves of a 64-bit value from lane l.
__device__ __forceinline__ unsigned long long shfl_u64(unsigned long long v, int l) {
  const uint32_t lo = __shfl((uint32_t)v, l);
  const uint32_t hi = __shfl((uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}

template <int LPT>
__global__ __launch_bounds__(256) void indexer_kernel(IndexArgs a) {
  __shared__ uint32_t hist[kBins / 2];
  __shared__ uint32_t blk_sh[kMaxTileTokens / kBlockTokens];
  __shared__ float sbuf[kMaxTileTokens];
  __shared__ uint32_t wmax[4];
  // This workgroup's share [r0, r1) of the flattened space, the units that
  // hold its first and last token (the units in between are consecutive),
  // and the first one's flattened start; derived by the first wave.
  __shared__ unsigned long long span_r[2];
  __shared__ unsigned long long span_off;
  __shared__ int span_u[2];
  __shared__ int span_len;  // length of the first unit
  using u64 = unsigned long long;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    u64 total = 0ull;
    for (int ub = 0; ub < a.units; ub += 64) total += wave_sum(padded_len(a, ub + lane));
    const u64 step = (u64)gridDim.x * kFlatAlign;
    const u64 share = (total + step - 1) / step * kFlatAlign;
    const u64 r0 = share * blockIdx.x;
    const u64 r1 = min(total, r0 + share);
    int uf = -1, ul = -1, len_f = 0;
    u64 off_f = 0ull;
    u64 run = 0ull;  // flattened start of unit ub
    for (int ub = 0; r0 < r1 && ub < a.units && ul < 0; ub += 64) {
      const int L = ub + lane < a.units ? unit_len(a, ub + lane) : 0;
      const u64 lp = padded(L);
      const u64 inc = wave_inclusive_scan(lp);
      const u64 off = run + inc - lp;
      const u64 m0 = __ballot(lp > 0ull && off <= r0 && r0 < off + lp);
      const u64 m1 = __ballot(lp > 0ull && off < r1 && r1 - 1 < off + lp);
      if (m0) {
        const int l = __ffsll((long long)m0) - 1;
        uf = ub + l;
        off_f = shfl_u64(off, l);
        len_f = __shfl(L, l);
      }
      if (m1) ul = ub + __ffsll((long long)m1) - 1;
      run += shfl_u64(inc, 63);
    }
    if (lane == 0) {
      span_r[0] = r0;
      span_r[1] = r1;
      span_off = off_f;
      span_u[0] = uf;
      span_u[1] = ul;
      span_len = len_f;
    }
  }
  __syncthreads();
  const u64 r0 = uniform_u64(span_r[0]);
  const u64 r1 = uniform_u64(span_r[1]);
  const int u_first = __builtin_amdgcn_readfirstlane(span_u[0]);
  const int u_last = __builtin_amdgcn_readfirstlane(span_u[1]);
  if (r0 >= r1 || u_first < 0) return;  // uniform over the workgroup
  u64 uoff = uniform_u64(span_off);
  for (int v = u_first; v <= u_last; ++v) {
    const int L = __builtin_amdgcn_readfirstlane(v == u_first ? span_len : unit_len(a, v));
    const u64 vlp = padded(L);
    const int lo = (int)((r0 > uoff ? r0 : uoff) - uoff);
    const int hi = min((int)((uoff + vlp < r1 ? uoff + vlp : r1) - uoff), L);
    for (int t0 = lo; t0 < hi; t0 += kMaxTileTokens)
      index_tile<LPT>(a, v, t0, min(hi, t0 + kMaxTileTokens), hist, blk_sh, sbuf, wmax);
    uoff += vlp;
  }
}

// Clears the per-unit histograms and maxima.
__global__ __launch_bounds__(256) void init_kernel(uint32_t* hist1, uint32_t* hist2,
                                                   uint32_t* maxkey, unsigned long long* hist1m,
                                                   unsigned long long* hist2m) {
  const int u = blockIdx.x;
  for (int i = threadIdx.x; i < kBins; i += 256) {
    hist1[(size_t)u * kBins + i] = 0u;
    hist2[(size_t)u * kBins + i] = 0u;
    if (hist1m) {
      hist1m[(size_t)u * kBins + i] = 0ull;
      hist2m[(size_t)u * kBins + i] = 0ull;
    }
  }
  if (threadIdx.x == 0) maxkey[u] = 0u;
}

// First-digit histogram and maximum of a caller-provided score array (the
// standalone selection entry point; the fused path gets both from stage 1).
__global__ __launch_bounds__(256) void score_hist_kernel(SelectArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wmax[4];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int L = unit_info(u, a.Hkv, a.NG, a.T, a.g, a.seq_lens, a.max_seq_len).L;
  const int c0 = c * kChunk;
  if (c0 >= L) return;
  const int c1 = min(L, c0 + kChunk);
  for (int i = threadIdx.x; i < kBins; i += 256) hist[i] = 0u;
  __syncthreads();
  const float* srow = a.scores + (size_t)u * a.score_ld;
  uint32_t kmax = 0u;
  for (int t = c0 + threadIdx.x; t < c1; t += 256) {
    const uint32_t key = order_key(srow[t]);
    atomicAdd(&hist[key >> kDigit1Shift], 1u);
    kmax = key > kmax ? key : kmax;
  }
  kmax = wave_max_u32(kmax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = kmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t mx = wmax[0];
    for (int w = 1; w < 4; ++w) mx = wmax[w] > mx ? wmax[w] : mx;
    atomicMax(&a.maxkey[u], mx);
  }
  for (int i = threadIdx.x; i < kBins; i += 256) {
    const uint32_t n = hist[i];
    if (n) atomicAdd(&a.hist1[(size_t)u * kBins + i], n);
  }
}

}  // namespace


// Workgroups of the indexer instance for `pair_count` that the current device
// holds at once (CUs x resident workgroups per CU), cached per device.
int indexer_resident_workgroups(int pair_count) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][5];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int slot = 0;
  while (slot < 4 && (4 << slot) != pair_count) ++slot;
  if (dev < kMaxDevices) {
    const int c = cache[dev][slot].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const void* fn = nullptr;
  switch (pair_count / 4) {
    case 1: fn = reinterpret_cast<const void*>(&indexer_kernel<1>); break;
    case 2: fn = reinterpret_cast<const void*>(&indexer_kernel<2>); break;
    case 4: fn = reinterpret_cast<const void*>(&indexer_kernel<4>); break;
    case 8: fn = reinterpret_cast<const void*>(&indexer_kernel<8>); break;
    case 16: fn = reinterpret_cast<const void*>(&indexer_kernel<16>); break;
    default: return 0;
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess) return 0;
  const int c = cus * per_cu;
  if (dev < kMaxDevices && c > 0) cache[dev][slot].store(c, std::memory_order_relaxed);
  return c;
}

hipError_t launch_init(uint32_t* hist1, uint32_t* hist2, uint32_t* maxkey,
                       unsigned long long* hist1m, unsigned long long* hist2m, int units,
                       hipStream_t stream) {
  init_kernel<<<units, 256, 0, stream>>>(hist1, hist2, maxkey, hist1m, hist2m);
  return hipGetLastError();
}

hipError_t launch_indexer(const IndexArgs& a, int units, hipStream_t stream) {
  if (units != a.units || a.workgroups < 1) return hipErrorInvalidValue;
  const dim3 grid(a.workgroups);
  switch (a.pair_count / 4) {
    case 1: indexer_kernel<1><<<grid, 256, 0, stream>>>(a); break;
    case 2: indexer_kernel<2><<<grid, 256, 0, stream>>>(a); break;
    case 4: indexer_kernel<4><<<grid, 256, 0, stream>>>(a); break;
    case 8: indexer_kernel<8><<<grid, 256, 0, stream>>>(a); break;
    case 16: indexer_kernel<16><<<grid, 256, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_hist(const SelectArgs& a, int units, hipStream_t stream) {
  score_hist_kernel<<<dim3(a.nchunk, units), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ssa

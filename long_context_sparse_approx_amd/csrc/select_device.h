// Chunk filter of the selection (internal to the library).
#pragma once

#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

constexpr int kNT = 256;             // threads per chunk workgroup
constexpr int kPer = kChunk / kNT;   // 16 consecutive tokens per thread

// The chunk filter's tail weight e^x (x <= 0): the hardware exp2 of
// t = x log2(e), with t carried past float32 precision (the product's rounding
// error, exact by a fused multiply-add, and the tail of the constant, added
// back as 2^t (1 + e ln 2)); within a few ulp of sexp(x), and 0 below -87
// like it.  It feeds the fp64 tail sum W (whose terms thus differ from the
// specified weights by a few ulp, well inside W's 1e-6 tolerance) and the
// necessary inclusion test, whose 2^-10 margin covers it; every decision
// that must match the oracle bit for bit uses sexp.
__device__ __forceinline__ float tail_exp(float x) {
  constexpr float kL2e = 0x1.715476p+0f;    // float32(log2 e)
  constexpr float kL2eLo = 0x1.4ae0c0p-26f;  // float32(log2 e - kL2e)
  constexpr float kLn2 = 0x1.62e430p-1f;    // float32(ln 2)
  const float t = x * kL2e;
  const float e = __builtin_fmaf(x, kL2e, -t) + x * kL2eLo;
  const float r = __builtin_amdgcn_exp2f(t);
  const float y = __builtin_fmaf(r * e, kLn2, r);
  return x < -87.0f ? 0.0f : y;
}

// Filter of chunk c of unit u = (b, grp, h) by a 256-thread workgroup.  s4
// holds the thread's 16 consecutive scores (entries at or past L are
// ignored); sh is the chunk's score buffer in LDS, of which the thread uses
// its own 16 entries; t1 is the unit's first-digit threshold and M its
// maximum score.  Writes the chunk's
// candidates (positions, keys and tail weights, second-digit histogram), its
// lists (tokens
// above the threshold digit, then tail tokens passing the necessary
// inclusion test fl(u * W_lb) < fl(m * w) with their weights), its
// candidate and list counts and its fp64 tail weight sum.
// Two passes over the thread's 16 tokens: the first computes every token's
// class, weight and inclusion test in groups of four (one Philox block each)
// and keeps only bit masks and the fp64 tail sum; after the scans the second
// visits the set bits only, recomputing the key and weight of the few tokens
// it writes.  Keeping no per-token arrays holds the kernel to 64 VGPRs, so a
// 1M-token layer's chunk workgroups are all resident at once.
__device__ __forceinline__ void filter_chunk(const SelectArgs& a, const SeqParams& p,
                                             const Thresh1& t1, float M, int u, int b, int h,
                                             int grp, int c, const float4 (&s4)[kPer / 4],
                                             float* sh, int* scan_scr, double* dscr) {
  const int c0 = c * kChunk;
  const int b1 = t1.b1;  // 2048 when there is no deterministic set
  // With top-p the stratum size is not known yet: list sampling candidates
  // whenever there is a budget.
  const bool sampling = p.m > 0 && (p.topp || p.L - p.k_eff > 0);
  const bool mass = t1.mode & kBoundMass;
  const float mf = (float)p.m;
  const uint64_t seed = a.seed[b];
  const int tb = threadIdx.x * kPer;
  const int nv = p.L - (c0 + tb);  // valid tokens of this thread: min(16, max(nv, 0))
  // Per-token class bits, formed arithmetically so that none of them is held
  // as a lane mask across the loop: d = first digit - b1 has its sign bit set
  // for a tail token (d < 0), and -d for a token above the threshold digit.
  // Positions past the sequence are scored -inf (weight exactly 0, so the
  // tail sum is unchanged) and their bits are cleared at the end.
  uint32_t tailbits = 0u, abovebits = 0u, sampbits = 0u;
  double wsum = 0.0;
  const uint32_t vmask = nv >= kPer ? 0xffffu : (nv <= 0 ? 0u : (1u << nv) - 1u);
  const bool ragged = c0 + kChunk > p.L;
  // The necessary test's left side u * W_lb as (word >> 8) * (W_lb 2^-24):
  // the same product, since both scalings by 2^-24 are exact, unless W_lb 2^-24
  // would be subnormal; then 0, which lists every token with a weight.
  const float wlb24 = t1.wlb >= 0x1.0p-100f ? t1.wlb * 0x1.0p-24f : 0.0f;
#pragma unroll
  for (int g = 0; g < kPer / 4; ++g) {
    // One group at a time: its loads may still be in flight while the
    // previous group is computed.  The empty asm ties the group's Philox
    // counter to the previous group's result, so the four blocks are not
    // computed at once (they would not fit 64 VGPRs).
    uint32_t jq = (uint32_t)(c0 + tb + 4 * g) >> 2;
    asm volatile("" : "+v"(jq) : "v"(sampbits));
    float s[4] = {s4[g].x, s4[g].y, s4[g].z, s4[g].w};
    // Kept for the second pass (no other thread reads this thread's entries).
    *reinterpret_cast<float4*>(sh + tb + 4 * g) = s4[g];
    if (ragged && nv < kPer) {  // ragged: uniform over the workgroup
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g + r >= nv) s[r] = -INFINITY;
    }
    uint4 wd = make_uint4(0u, 0u, 0u, 0u);
    if (sampling) wd = philox_block(seed, b, h, jq, grp);
    const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      const int d = (int)(order_key(s[r]) >> kDigit1Shift) - b1;
      const uint32_t tbit = (uint32_t)d >> 31;
      tailbits |= tbit << i;
      abovebits |= ((uint32_t)(-d) >> 31) << i;
      const float w = tail_exp(s[r] - M);
      wsum += (double)__uint_as_float(__float_as_uint(w) & (0u - tbit));
      const uint32_t sbit = (float)(words[r] >> 8) * wlb24 < mf * w ? 1u : 0u;
      sampbits |= (sbit & tbit) << i;
    }
  }
  const uint32_t abovemask = abovebits & vmask;
  const uint32_t candmask = ~(abovebits | tailbits) & vmask;
  const uint32_t sampmask = sampling ? sampbits & vmask : 0u;
  int total;
  const int off = block_exclusive_scan<kNT>(__popc(candmask), scan_scr, &total);
  int lst_tot;
  const int lst = block_exclusive_scan<kNT>(__popc(abovemask) | (__popc(sampmask) << 16),
                                            scan_scr, &lst_tot);
  const int n_above = lst_tot & 0xffff;
  int32_t* cidx = a.cand_idx + (size_t)u * a.seg_ld + c0;
  uint32_t* ckey = a.cand_key + (size_t)u * a.seg_ld + c0;
  float* cw = a.cand_w + (size_t)u * a.seg_ld + c0;
  int32_t* lidx = a.list_idx + (size_t)u * a.seg_ld + c0;
  float* lw = a.list_w + (size_t)u * a.seg_ld + c0;
  int wc = off, wa = lst & 0xffff, ws = n_above + (lst >> 16);
  // The classes are disjoint; ascending bits keep every list in index order.
  for (uint32_t rest = candmask | abovemask | sampmask; rest != 0u; rest &= rest - 1u) {
    const int i = __builtin_ctz(rest);
    const uint32_t bit = 1u << i;
    const int t = c0 + tb + i;
    const float s = sh[tb + i];
    if (candmask & bit) {
      const uint32_t key = order_key(s);
      const float w = sexp(s - M);
      cidx[wc] = t;
      ckey[wc] = key;
      cw[wc] = w;
      ++wc;
      const int d2 = (key >> kDigit2Shift) & (kBins - 1);
      atomicAdd(&a.hist2[(size_t)u * kBins + d2], 1u);
      if (mass) atomicAdd(&a.hist2m[(size_t)u * kBins + d2], mass_units(w));
    } else if (abovemask & bit) {
      lidx[wa++] = t;
    } else {
      lidx[ws] = t;
      lw[ws] = sexp(s - M);
      ++ws;
    }
  }
  const double wtot = block_sum_f64<kNT>(wsum, dscr);
  if (threadIdx.x == 0) {
    const size_t ci = (size_t)u * a.nchunk + c;
    a.cand_cnt[ci] = total;
    a.wpart[ci] = wtot;
    a.list_cnt[2 * ci] = n_above;
    a.list_cnt[2 * ci + 1] = lst_tot >> 16;
  }
}

}  // namespace ssa

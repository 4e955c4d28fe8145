// Chunk filter of the selection (internal to the library).
#pragma once

#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

constexpr int kNT = 256;             // threads per chunk workgroup
constexpr int kPer = kChunk / kNT;   // 16 consecutive tokens per thread
constexpr int kStage = 128;          // second-pass entries a wave stages in LDS

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

// ---- First-pass building blocks.  A token's class and test results are
// shifted into per-thread 16-bit accumulators, token by token
// (acc <- 2 acc + bit, first token ending in bit 15): one compare, whose lane
// mask is the carry-in of an add with carry, per bit.

// acc <- 2 acc + [a < b], unsigned, b uniform over the wave.  Also returns w
// where a < b and 0 elsewhere.
__device__ __forceinline__ float push_lt_keep(uint32_t& acc, uint32_t a, uint32_t b, float w) {
  float r;
  asm("v_cmp_gt_u32_e32 vcc, %[b], %[a]\n\t"
      "v_cndmask_b32_e32 %[r], 0, %[w], vcc\n\t"
      "v_addc_co_u32_e32 %[acc], vcc, %[acc], %[acc], vcc"
      : [acc] "+v"(acc), [r] "=&v"(r)
      : [a] "v"(a), [b] "s"(b), [w] "v"(w)
      : "vcc");
  return r;
}

// acc <- 2 acc + [a > b], unsigned, b uniform over the wave.
__device__ __forceinline__ uint32_t push_gt(uint32_t acc, uint32_t a, uint32_t b) {
  asm("v_cmp_lt_u32_e32 vcc, %[b], %[a]\n\t"
      "v_addc_co_u32_e32 %[acc], vcc, %[acc], %[acc], vcc"
      : [acc] "+v"(acc)
      : [a] "v"(a), [b] "s"(b)
      : "vcc");
  return acc;
}

// acc <- 2 acc + [float(word) <= y] (false when y is NaN).
__device__ __forceinline__ uint32_t push_word_le(uint32_t acc, uint32_t word, float y) {
  float f;
  asm("v_cvt_f32_u32_e32 %[f], %[word]\n\t"
      "v_cmp_ge_f32_e32 vcc, %[y], %[f]\n\t"
      "v_addc_co_u32_e32 %[acc], vcc, %[acc], %[acc], vcc"
      : [acc] "+v"(acc), [f] "=&v"(f)
      : [word] "v"(word), [y] "v"(y)
      : "vcc");
  return acc;
}

// a ^ b ^ k in one v_bitop3_b32 (k uniform over the wave).
__device__ __forceinline__ uint32_t xor3_uniform(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) for a key that is uniform
// over the wave: the same rounds as philox4x32_10, with each round's two
// three-way exclusive ors as single instructions.  The first round, whose
// counter words c1 and c3 are uniform too, is left to the compiler.
__device__ __forceinline__ uint4 philox4x32_10_uniform_key(uint4 c, uint32_t k0, uint32_t k1) {
  {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1,
                   (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
#pragma unroll
  for (int i = 1; i < 10; ++i) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4(xor3_uniform((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1,
                   xor3_uniform((uint32_t)(p0 >> 32), c.w, k1), (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The words of philox_block (counter (jq, h, b, grp), key = the seed) with a
// uniform seed.
__device__ __forceinline__ uint4 philox_block_uniform_key(uint64_t seed, int b, int h,
                                                          uint32_t jq, int grp) {
  return philox4x32_10_uniform_key(make_uint4(jq, (uint32_t)h, (uint32_t)b, (uint32_t)grp),
                                   (uint32_t)seed, (uint32_t)(seed >> 32));
}

// The first digit of order_key(s) (its top 11 bits).
__device__ __forceinline__ uint32_t first_digit(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t m = (uint32_t)((int32_t)u >> 31) | 0x80000000u;
  return (u ^ m) >> kDigit1Shift;
}

struct FirstPass {
  uint32_t tail, above, samp;  // token i of the thread in bit 15 - i
  double wsum;                 // fp64 sum of the tail tokens' weights
};

// The filter's first pass over a thread's 16 consecutive tokens, in groups
// of four (one Philox block each): the class of every token (first digit
// below b1: tail; above b1: listed as deterministic; equal: candidate), the
// fp64 sum of the tail weights, and the necessary inclusion test.  With the
// final test fl(u W) < fl(m w) (u = (word >> 8) 2^-24) and W_lb <= W (1 -
// 2^-10), any token the final test includes has word < z 2^32 (1 - 2^-11) +
// 256, z = m w_f / W_lb and w_f this pass's weight (within a few ulp of the
// specified one); the test word <= fl(w_f K + 512) with K = fl(m 2^32 / W_lb)
// (compared in float32) holds for every such word, the rounding of K, of the
// product and of the word's conversion being inside the 2^-11 and +256
// margins.  K = inf (W_lb = 0, or too small) lists every token with a weight.
// Ragged: positions at or past the thread's nv valid tokens are scored -inf
// (weight 0); their bits are cleared by the caller.
template <bool kRagged>
__device__ __forceinline__ FirstPass filter_first_pass(const float4 (&s4)[kPer / 4], float* sh,
                                                       int tb, int c0, int nv, float M,
                                                       uint32_t b1, float K, bool sampling,
                                                       uint64_t seed, int b, int h, int grp) {
  uint32_t tail = 0u, above = 0u, samp = 0u;
  double wsum = 0.0;
#pragma unroll
  for (int g = 0; g < kPer / 4; ++g) {
    // One group at a time: its loads may still be in flight while the
    // previous group is computed.  The empty asm ties the group's Philox
    // counter to the previous group's result, so the four blocks are not
    // computed at once (they would not fit 64 VGPRs).
    uint32_t jq = (uint32_t)(c0 + tb + 4 * g) >> 2;
    asm volatile("" : "+v"(jq) : "v"(samp));
    float s[4] = {s4[g].x, s4[g].y, s4[g].z, s4[g].w};
    // Kept for the second pass (no other thread reads this thread's entries).
    *reinterpret_cast<float4*>(sh + tb + 4 * g) = s4[g];
    if (kRagged) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g + r >= nv) s[r] = -INFINITY;
    }
    uint4 wd = make_uint4(0u, 0u, 0u, 0u);
    if (sampling) wd = philox_block_uniform_key(seed, b, h, jq, grp);
    const uint32_t words[4] = {wd.x, wd.y, wd.z, wd.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t d = first_digit(s[r]);
      const float w = tail_exp(s[r] - M);
      wsum += (double)push_lt_keep(tail, d, b1, w);
      above = push_gt(above, d, b1);
      samp = push_word_le(samp, words[r], __builtin_fmaf(w, K, 512.0f));
    }
  }
  return FirstPass{tail, above, samp, wsum};
}

// Filter of chunk c of unit u = (b, grp, h) by a 256-thread workgroup.  s4
// holds the thread's 16 consecutive scores (entries at or past L are
// ignored); sh is the chunk's score buffer in LDS, of which the thread uses
// its own 16 entries; t1 is the unit's first-digit threshold and M its
// maximum score.  Writes the chunk's
// candidates (positions, keys and tail weights, second-digit histogram), its
// lists (tokens
// above the threshold digit, then tail tokens passing the necessary
// inclusion test of filter_first_pass, with their weights), its candidate
// and list counts and its fp64 tail weight sum.
// Two passes over the thread's 16 tokens: the first computes every token's
// class, weight and inclusion test in groups of four (one Philox block each)
// and keeps only bit masks and the fp64 tail sum; after the scans the second
// visits the set bits only, recomputing the key and weight of the few tokens
// it writes.  Keeping no per-token arrays holds the kernel to 64 VGPRs, so a
// 1M-token layer's chunk workgroups are all resident at once.
__device__ __forceinline__ void filter_chunk(const SelectArgs& a, const SeqParams& p,
                                             const Thresh1& t1, float M, int u, int b, int h,
                                             int grp, int c, const float4 (&s4)[kPer / 4],
                                             float* sh, int* scan_scr, double* dscr,
                                             uint32_t* stage) {
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
  const uint32_t vmask = nv >= kPer ? 0xffffu : (nv <= 0 ? 0u : (1u << nv) - 1u);
  // Only the chunk holding the sequence's end has positions past it.
  const bool ragged = c0 + kChunk > p.L;
  const float K = t1.wlb > 0.0f ? (mf * 0x1.0p32f) / t1.wlb : INFINITY;
  const FirstPass fp =
      ragged ? filter_first_pass<true>(s4, sh, tb, c0, nv, M, (uint32_t)b1, K, sampling, seed, b,
                                       h, grp)
             : filter_first_pass<false>(s4, sh, tb, c0, nv, M, (uint32_t)b1, K, sampling, seed,
                                        b, h, grp);
  // Bit i for token i.
  const uint32_t tailbits = __builtin_bitreverse32(fp.tail) >> 16;
  const uint32_t abovebits = __builtin_bitreverse32(fp.above) >> 16;
  const uint32_t sampbits = __builtin_bitreverse32(fp.samp) >> 16;
  const double wsum = fp.wsum;
  const uint32_t abovemask = abovebits & vmask;
  const uint32_t candmask = ~(abovebits | tailbits) & vmask;
  const uint32_t sampmask = sampling ? sampbits & tailbits & vmask : 0u;
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
  // One entry: its token (offset ti in the chunk), class (0 candidate, 1 above
  // the threshold digit, 2 listed tail token) and slot in its list.
  auto emit = [&](int ti, int cls, int out) {
    const int t = c0 + ti;
    const float s = sh[ti];
    if (cls == 0) {
      const uint32_t key = order_key(s);
      const float w = sexp(s - M);
      cidx[out] = t;
      ckey[out] = key;
      cw[out] = w;
      const int d2 = (key >> kDigit2Shift) & (kBins - 1);
      atomicAdd(&a.hist2[(size_t)u * kBins + d2], 1u);
      if (mass) atomicAdd(&a.hist2m[(size_t)u * kBins + d2], mass_units(w));
    } else if (cls == 1) {
      lidx[out] = t;
    } else {
      lidx[out] = t;
      lw[out] = sexp(s - M);
    }
  };
  // The classes are disjoint; ascending bits keep every list in index order.
  // The wave's entries are staged (token, class and slot packed in a word) so
  // that each lane then emits one of them: one round for the usual few dozen,
  // instead of as many rounds as the busiest lane has entries.
  const uint32_t rest0 = candmask | abovemask | sampmask;
  const int nmine = __popc(rest0);
  const int incl = wave_inclusive_scan<int>(nmine);
  const int q_total = __builtin_amdgcn_readlane(incl, 63);
  int wc = off, wa = lst & 0xffff, ws = n_above + (lst >> 16);
  // Class and slot of the entry at bit i, counted in each class's list.
#define SSA_NEXT_SLOT(i, cls, out)                             \
  const uint32_t bit_ = 1u << (i);                             \
  const bool isc_ = (candmask & bit_) != 0u;                   \
  const bool isa_ = !isc_ && (abovemask & bit_) != 0u;         \
  const int cls = isc_ ? 0 : (isa_ ? 1 : 2);                   \
  const int out = isc_ ? wc : (isa_ ? wa : ws);                \
  wc += isc_ ? 1 : 0;                                          \
  wa += isa_ ? 1 : 0;                                          \
  ws += (!isc_ && !isa_) ? 1 : 0
  if (q_total <= kStage) {  // uniform over the wave
    int k = incl - nmine;
    for (uint32_t r = rest0; r != 0u; r &= r - 1u) {
      const int i = __builtin_ctz(r);
      SSA_NEXT_SLOT(i, cls, out);
      stage[k++] = (uint32_t)(tb + i) | ((uint32_t)cls << 12) | ((uint32_t)out << 14);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int j = (int)(threadIdx.x & 63); j < q_total; j += 64) {
      const uint32_t e = stage[j];
      emit((int)(e & 4095u), (int)((e >> 12) & 3u), (int)(e >> 14));
    }
  } else {
    for (uint32_t r = rest0; r != 0u; r &= r - 1u) {
      const int i = __builtin_ctz(r);
      SSA_NEXT_SLOT(i, cls, out);
      emit(tb + i, cls, out);
    }
  }
#undef SSA_NEXT_SLOT
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

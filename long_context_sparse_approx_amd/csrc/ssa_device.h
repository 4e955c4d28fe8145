// Device-side building blocks of the stratified sparse decode path (gfx950).
//
// Shared by the kernels in this directory only.  Everything here is written
// for 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssa.h"
#include "ssa_launch.h"

namespace ssa {

constexpr int kBlockTokens = SSA_BLOCK_TOKENS;
constexpr int kChunk = SSA_CHUNK_TOKENS;
constexpr int kWave = 64;
// Radix digits of the 32-bit order key: 11 + 11 + 10 bits.
constexpr int kDigit1Shift = 21;
constexpr int kDigit2Shift = 10;
constexpr int kBins = 2048;
constexpr int kBins3 = 1024;

// Per-unit (batch, kv head) selection state written by the resolve stage.
enum : int32_t {
  kFlagEmpty = 1,     // L == 0: nothing to read
  kFlagDense = 2,     // k + m >= L: every token, weight 1
  kFlagNoTopk = 4,    // k == 0: every token is in the tail
  kFlagSample = 8,    // Poisson sampling of the tail is active
};

struct UnitState {
  uint32_t tkey;        // order key of the stratum's last (k-th) token
  int32_t ties_needed;  // tokens with key == tkey that join the deterministic set
  float M;              // maximum score of the sequence
  float W;              // tail normaliser used for sampling
  int32_t flags;
  int32_t k_eff;        // size k of the deterministic stratum
  int32_t m;
  int32_t L;
};
static_assert(sizeof(UnitState) == 32, "the host reserves 32 bytes per unit");

// Refine mode: a member's selection state.  The member's stratum is the
// candidates whose word ((~own key) << 24) | position is at most vstar.
struct MemberState {
  unsigned long long vstar;
  float W;     // the member's tail normaliser
  float M;     // the group's maximum proxy score
  int32_t k;   // the member's stratum size
  int32_t flags;
  int32_t L;   // the member's span
  int32_t m;
};
static_assert(sizeof(MemberState) == 32, "the host reserves 32 bytes per member unit");

// ---------------------------------------------------------------- sizes

__device__ __forceinline__ int clamp_len(int L, int max_seq_len) {
  return L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
}

__device__ __forceinline__ int clamp_count(int n, int cap) {
  return n < 0 ? 0 : (n > cap ? cap : n);
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------- ranking

// Monotone float -> uint32 map: larger float, larger key; -0.0 just below +0.0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- exp

// The specified float32 exp used for tail weights (x <= 0): Cody-Waite
// reduction x = n ln2 + r (ln2 split into a 16-fractional-bit head and a
// float32 tail), degree-7 Taylor polynomial of e^r in Horner form, then an
// exact scale by 2^n.  One rounding per operation, no fused multiply-add,
// 0 for x < -87 (so every non-zero result is a normal float).  Both ranking
// decisions that depend on it must be reproducible bit for bit off the GPU.
__device__ __forceinline__ float sexp(float x) {
#pragma clang fp contract(off)
  const float kLog2e = 0x1.715476p+0f;   // float32(1 / ln 2)
  const float kLn2Hi = 0x1.62e4p-1f;     // floor(ln2 * 2^16) / 2^16
  const float kLn2Lo = 0x1.7f7d1cp-20f;  // float32(ln2 - head)
  const bool low = x < -87.0f;
  const float xs = low ? 0.0f : x;
  const float n = __builtin_rintf(xs * kLog2e);
  float r = xs - n * kLn2Hi;
  r = r - n * kLn2Lo;
  float p = 0x1.a01a02p-13f;             // 1/7!
  p = p * r + 0x1.6c16c2p-10f;           // 1/6!
  p = p * r + 0x1.111112p-7f;            // 1/5!
  p = p * r + 0x1.555556p-5f;            // 1/4!
  p = p * r + 0x1.555556p-3f;            // 1/3!
  p = p * r + 0.5f;                      // 1/2!
  p = p * r + 1.0f;                      // 1/1!
  p = p * r + 1.0f;                      // 1/0!
  const float y = __builtin_ldexpf(p, (int)n);
  return low ? 0.0f : y;
}

// ---------------------------------------------------------------- lane butterflies

// The partner lane across lane-index bit BIT of a 16-lane row (DPP: quad
// permutations for bits 0 and 1, the half-row mirror for bit 2, a rotation
// by 8 for bit 3).  Each pairing is an involution that joins the two halves
// of the current group, so the butterfly sums neighbouring slices first.
template <int BIT>
__device__ __forceinline__ float dpp_partner(float x) {
  constexpr int ctrl = BIT == 0 ? 0xB1 : (BIT == 1 ? 0x4E : (BIT == 2 ? 0x141 : 0x128));
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               ctrl, 0xf, 0xf, false));
}

// Sum of the LPT (<= 16, a power of two) lanes of an aligned lane group,
// pairwise: neighbouring lanes first, then neighbouring pairs, and so on;
// every lane of the group ends with the same sum.
template <int LPT>
__device__ __forceinline__ float butterfly(float p) {
  if constexpr (LPT >= 2) p = p + dpp_partner<0>(p);
  if constexpr (LPT >= 4) p = p + dpp_partner<1>(p);
  if constexpr (LPT >= 8) p = p + dpp_partner<2>(p);
  if constexpr (LPT >= 16) p = p + dpp_partner<3>(p);
  return p;
}

// ---------------------------------------------------------------- top-p mass

// Approximate mass of a token in integer units: floor(w * 2^38) for a weight
// w = sexp(s - M) in [0, 1].  The scaling by a power of two is exact and the
// conversion truncates, so this is an exact floor; integer sums of these
// units do not depend on their order.
constexpr int kMassShift = 38;
__device__ __forceinline__ unsigned long long mass_units(float w) {
  return (unsigned long long)(w * 0x1.0p38f);
}

// ceil(p * Q) exactly, p clamped to [0, 1] (NaN as 0), Q < 2^62.
// p = f * 2^e with f in [0.5, 1), so p * Q = (f * 2^24) * Q / 2^(24 - e) with
// an integer numerator below 2^86.
__device__ __forceinline__ unsigned long long mass_target(float p, unsigned long long Q) {
  if (!(p > 0.0f)) return 0ull;
  if (p >= 1.0f) return Q;
  int e;
  const float f = __builtin_frexpf(p, &e);
  const unsigned long long mant = (unsigned long long)(f * 0x1.0p24f);  // exact, < 2^24
  const unsigned __int128 num = (unsigned __int128)mant * Q;
  const int sh = 24 - e;  // >= 25 for p < 1
  if (sh >= 120) return num != 0 ? 1ull : 0ull;  // p * Q < 2^86 / 2^120 < 1
  const unsigned __int128 den = (unsigned __int128)1 << sh;
  return (unsigned long long)((num + den - 1) >> sh);
}

// ---------------------------------------------------------------- Philox

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// -> 64-bit multiplies with the round function
//   (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
// and a Weyl bump of the key between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;  // one v_mad_u64_u32 each
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1,
                   (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The four words for tokens 4*jq .. 4*jq+3 of (b, h, query group grp):
// counter (jq, h, b, grp), key = the 64-bit seed, low word first.
__device__ __forceinline__ uint4 philox_block(uint64_t seed, int b, int h, uint32_t jq,
                                              int grp) {
  return philox4x32_10(make_uint4(jq, (uint32_t)h, (uint32_t)b, (uint32_t)grp), (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}

__device__ __forceinline__ float uniform24(uint32_t word) {
  return (float)(word >> 8) * 0x1.0p-24f;
}

// ---------------------------------------------------------------- reductions

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Maximum over the wave: the running maximum of the DPP pattern below (the
// same steps as the inclusive scan), read from the last lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto step = [](uint32_t x, uint32_t o) { return o > x ? o : x; };
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over the 64 lanes of a wave (int or 64-bit unsigned).
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

template <>
__device__ __forceinline__ int wave_inclusive_scan<int>(int v);

// 32-bit integer sum over the wave: the DPP inclusive scan's last lane.
template <>
__device__ __forceinline__ int wave_sum<int>(int v) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan<int>(v), 63);
}

// 32-bit integers: six DPP adds in the VALU instead of six LDS-crossbar
// shuffles.  Within each 16-lane row: add the value 1, 2, 4 and 8 lanes
// below (lanes without one add 0); then row 1 and row 3 add the last lane of
// the row below (row_bcast:15), rows 2 and 3 the last lane of row 1
// (row_bcast:31).
template <>
__device__ __forceinline__ int wave_inclusive_scan<int>(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

template <typename T>
struct same_type {
  using type = T;
};

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64);
// `scratch` holds NT/64 values in LDS.  Returns the exclusive prefix and
// writes the block total to *total.  Contains two barriers.  The value type
// is taken from the scratch array.
template <int NT, typename T>
__device__ __forceinline__ T block_exclusive_scan(typename same_type<T>::type v, T* scratch,
                                                  T* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const T inc = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const T s = scratch[w];
    base += (w < wave) ? s : (T)0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Deterministic block sum of doubles (fixed tree order); result in every thread.
template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* scratch) {
  constexpr int NW = NT / 64;
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

template <int NT>
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v,
                                                            unsigned long long* scratch) {
  constexpr int NW = NT / 64;
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  unsigned long long t = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

template <int NT>
__device__ __forceinline__ int block_sum_i32(int v, int* scratch) {
  constexpr int NW = NT / 64;
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

// Given a histogram `hist` of `nbins` bins in LDS and a target k >= 1 (a rank
// for counts, mass units for masses), find the bin b* with
// sum(bins > b*) < k <= sum(bins >= b*), and the remainder k - sum(bins > b*).
// Bins are scanned from the top.  Every thread of the NT-thread block must
// call it; the answer is returned in every thread.  T is uint32_t (counts,
// summed as int) or unsigned long long (mass units).
template <int NT, typename H, typename T>
__device__ __forceinline__ void find_bin(const H* hist, int nbins, typename same_type<T>::type k,
                                         T* scan_scratch,
                                         T* out_pair, int* bin_out, T* rem_out) {
  const int per = nbins / NT;  // bins per thread (nbins is a multiple of NT)
  const int top = nbins - 1 - threadIdx.x * per;  // this thread's highest bin
  T mine = 0;
  for (int i = 0; i < per; ++i) mine += (T)hist[top - i];
  T total;
  const T before = block_exclusive_scan<NT>(mine, scan_scratch, &total);
  if (before < k && k <= before + mine) {
    T run = before;
    for (int i = 0; i < per; ++i) {
      const T c = (T)hist[top - i];
      if (run + c >= k) {
        out_pair[0] = (T)(top - i);
        out_pair[1] = k - run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  *bin_out = (int)out_pair[0];
  *rem_out = out_pair[1];
  __syncthreads();
}

template <int NT>
__device__ __forceinline__ void find_rank_bin(const uint32_t* hist, int nbins, int k,
                                              int* scan_scratch, int* out_pair, int* bin_out,
                                              int* rem_out) {
  find_bin<NT>(hist, nbins, k, scan_scratch, out_pair, bin_out, rem_out);
}

// Sum of the counts of the bins above `bin` (every thread of the block calls).
template <int NT>
__device__ __forceinline__ int count_above(const uint32_t* hist, int nbins, int bin, int* scratch) {
  int v = 0;
  for (int i = bin + 1 + (int)threadIdx.x; i < nbins; i += NT) v += (int)hist[i];
  return block_sum_i32<NT>(v, scratch);
}

// The same two searches by one wave (all 64 lanes call; no barrier).  Lane l
// sums its per = nbins / 64 bins from the top (top - l * per down), a wave
// scan finds the lane where the running sum reaches k, and a second scan over
// that lane's bins, one per lane, finds the bin.  A k beyond the histogram's
// total ends at bin 0 (remainder k - sum(bins > 0)).  The result is in every
// lane.  nbins is a multiple of 64 and at most 64 * 64.
template <typename T, typename H>
__device__ __forceinline__ void wave_find_bin(const H* hist, int nbins, T k, int* bin_out,
                                              T* rem_out) {
  const int lane = threadIdx.x & 63;
  const int per = nbins >> 6;
  const int top = nbins - 1 - lane * per;
  T mine = 0;
  for (int i = 0; i < per; ++i) mine += (T)hist[top - i];
  const T inc = wave_inclusive_scan<T>(mine);
  const unsigned long long hit = __ballot(inc >= k);
  const int l = hit ? __builtin_ctzll(hit) : 63;
  const T before = __shfl(inc - mine, l);  // the bins above lane l's
  const int top_l = nbins - 1 - l * per;
  const T c = lane < per ? (T)hist[top_l - lane] : (T)0;
  const T inc2 = wave_inclusive_scan<T>(c) + before;
  const unsigned long long hit2 = __ballot(lane < per && inc2 >= k);
  const int i = hit2 ? __builtin_ctzll(hit2) : per - 1;
  *bin_out = top_l - i;
  *rem_out = k - __shfl(inc2 - c, i);
}

__device__ __forceinline__ int wave_count_above(const uint32_t* hist, int nbins, int bin) {
  int v = 0;
  for (int i = bin + 1 + (int)(threadIdx.x & 63); i < nbins; i += 64) v += (int)hist[i];
  return wave_sum<int>(v);
}

// Where the stratum ends at one radix digit, given the open bounds `mode`:
// the count bound ends in bin bc with remainder rc, the mass bound in bin bm
// with remainder rm.  The bound reached first (the higher bin, as keys are
// visited from the top) decides; both stay open when they share the bin.
struct DigitBound {
  int bin;
  int rem;
  unsigned long long rem_mass;
  int mode;
};

__device__ __forceinline__ DigitBound combine_bounds(int mode, int bc, int rc, int bm,
                                                     unsigned long long rm) {
  if (mode == kBoundCount || (mode == (kBoundCount | kBoundMass) && bc > bm))
    return DigitBound{bc, rc, 0ull, kBoundCount};
  if (mode == kBoundMass || bm > bc) return DigitBound{bm, 0, rm, kBoundMass};
  return DigitBound{bc, rc, rm, kBoundCount | kBoundMass};
}

// A selection unit: (sequence b, query group grp, kv head h), numbered
// u = (b * NG + grp) * Hkv + h.  With T query positions per sequence (the last
// T of its P cached tokens) and groups of g consecutive queries, the unit's
// span is the causal length of the group's last member.
struct UnitInfo {
  int b, grp, h, L;
};

__device__ __forceinline__ int member_span(int P, int T, int t) {
  const int L = P - T + t + 1;
  return L < 0 ? 0 : L;
}

__device__ __forceinline__ UnitInfo unit_info(int u, int Hkv, int NG, int T, int g,
                                              const int32_t* seq_lens, int max_seq_len) {
  UnitInfo r;
  const int bg = u / Hkv;
  r.h = u - bg * Hkv;
  r.b = bg / NG;
  r.grp = bg - r.b * NG;
  const int last = min((r.grp + 1) * g, T) - 1;
  r.L = member_span(clamp_len(seq_lens[r.b], max_seq_len), T, last);
  return r;
}

// Selection parameters of a unit as the kernels read them.  k_eff is the
// count bound min(topk, L).  With a top-p mass the stratum may end earlier,
// so only m >= L makes the unit dense before the selection is resolved.
struct SeqParams {
  int L, k_eff, m;
  bool dense;
  bool topp;
  float p;
};

__device__ __forceinline__ SeqParams seq_params(int L, const int32_t* topk, const float* top_p,
                                                const int32_t* sample_budget, int b,
                                                int max_topk, int kmult = 1) {
  SeqParams p;
  p.L = L;
  // The three loads are unconditional (without a top-p array the last one
  // reads the budget's word and is discarded), so they go out together.
  const int tk = topk[b];
  const int mb = sample_budget[b];
  float pv;
  __builtin_memcpy(&pv, top_p ? static_cast<const void*>(top_p + b)
                              : static_cast<const void*>(sample_budget + b), sizeof(float));
  const int64_t k64 = (int64_t)min(max(tk, 0), max_topk) * kmult;
  const int k = k64 > L ? L : (int)k64;
  p.m = max(mb, 0);
  p.topp = top_p != nullptr;
  p.p = p.topp ? pv : 1.0f;
  // Both rules evaluated and selected without a branch, so the caller's
  // loads that follow stay in one basic block with these.
  const bool dense_m = p.m >= p.L;
  const bool dense_km = (int64_t)k + (int64_t)p.m >= (int64_t)p.L;
  p.dense = (p.topp & dense_m) | (!p.topp & dense_km);
  p.k_eff = min(k, p.L);
  return p;
}

}  // namespace ssa

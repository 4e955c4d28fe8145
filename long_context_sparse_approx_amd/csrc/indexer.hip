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
// for 32 pairs at d = 128).  LPT lanes cover one token with one 16-byte load
// each; a wave instruction therefore reads 64/LPT token slices and every lane
// keeps UNR independent loads in flight.  The fp32 proxy query (scaled) lives
// in registers; the products are exact bf16 x fp32 -> fp32 with fp32
// accumulation.  The epilogue writes the score, counts the score's first
// radix digit (top 11 bits of the order key) in an LDS histogram and tracks
// the maximum order key; both are flushed with integer atomics, so the result
// is independent of scheduling.
#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

namespace {

// Largest token tile of one indexer workgroup (its block ids are staged in LDS).
constexpr int kMaxTileTokens = 8192;

__device__ __forceinline__ float dot8(const float* qb, uint4 v) {
  float s = qb[0] * bf16_lo(v.x);
  s = __builtin_fmaf(qb[1], bf16_hi(v.x), s);
  s = __builtin_fmaf(qb[2], bf16_lo(v.y), s);
  s = __builtin_fmaf(qb[3], bf16_hi(v.y), s);
  s = __builtin_fmaf(qb[4], bf16_lo(v.z), s);
  s = __builtin_fmaf(qb[5], bf16_hi(v.z), s);
  s = __builtin_fmaf(qb[6], bf16_lo(v.w), s);
  s = __builtin_fmaf(qb[7], bf16_hi(v.w), s);
  return s;
}

template <int LPT>
__global__ __launch_bounds__(256) void indexer_kernel(IndexArgs a) {
  constexpr int TPI = kWave / LPT;      // tokens per wave-wide load
  constexpr int UNR = 8;                // loads in flight per lane
  constexpr int WAVE_TOK = TPI * UNR;   // tokens per wave per iteration
  constexpr int WG_TOK = 4 * WAVE_TOK;  // tokens per workgroup per iteration
  __shared__ float qsh[16 * 128];
  __shared__ uint32_t hist[kBins];
  __shared__ int blk_sh[kMaxTileTokens / kBlockTokens];
  __shared__ uint32_t wmax[4];

  const int u = blockIdx.y;
  const int b = u / a.Hkv;
  const int h = u - b * a.Hkv;
  const int L = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int t0 = blockIdx.x * a.tokens_per_wg;
  if (t0 >= L) return;  // uniform over the workgroup
  const int t_end = min(L, t0 + a.tokens_per_wg);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nd = 2 * a.pair_count;

  // Stage the query group's scored slice and the tile's block ids in LDS.
  for (int i = tid; i < a.G * nd; i += 256) {
    const int g = i / nd;
    const int e = i - g * nd;
    const uint16_t bits =
        a.q[(size_t)(b * a.Hq + h * a.G + g) * a.d + 2 * a.pair_begin + e];
    qsh[i] = __uint_as_float((uint32_t)bits << 16);
  }
  const int blk0 = t0 / kBlockTokens;
  const int nblk = (t_end - t0 + kBlockTokens - 1) / kBlockTokens;
  const int* btrow = a.block_table + (size_t)b * a.max_blocks;
  for (int i = tid; i < nblk; i += 256) {
    int blk = btrow[blk0 + i];
    blk_sh[i] = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
  }
  for (int i = tid; i < kBins; i += 256) hist[i] = 0u;
  __syncthreads();
  // Per-lane proxy query: qb = (scale / G) * sum_g q_g over this lane's 8 dims.
  const int sub = lane % LPT;
  float qb[8];
  const float qscale = a.scale / (float)a.G;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float s = 0.0f;
    for (int g = 0; g < a.G; ++g) s += qsh[g * nd + sub * 8 + i];
    qb[i] = s * qscale;
  }

  const size_t blk_stride = (size_t)a.Hkv * kBlockTokens * a.d;
  const uint16_t* kbase = a.k_cache + (size_t)h * kBlockTokens * a.d + 2 * a.pair_begin + sub * 8;
  float* srow = a.scores + (size_t)u * a.score_ld;
  uint32_t kmax = 0u;

  for (int base = t0 + wave * WAVE_TOK; base < t_end; base += WG_TOK) {
    uint4 kv[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int t = base + r * TPI + lane / LPT;
      kv[r] = make_uint4(0u, 0u, 0u, 0u);
      if (t < t_end) {
        const int blk = blk_sh[(t - t0) >> 4];
        kv[r] = *reinterpret_cast<const uint4*>(kbase + (size_t)blk * blk_stride +
                                                (size_t)(t & 15) * a.d);
      }
    }
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      float s = dot8(qb, kv[r]);
#pragma unroll
      for (int off = LPT / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      const int t = base + r * TPI + lane / LPT;
      if (sub == 0 && t < t_end) {
        srow[t] = s;
        const uint32_t key = order_key(s);
        atomicAdd(&hist[key >> kDigit1Shift], 1u);
        kmax = key > kmax ? key : kmax;
      }
    }
  }

  kmax = wave_max_u32(kmax);
  if (lane == 0) wmax[wave] = kmax;
  __syncthreads();
  if (tid == 0) {
    uint32_t mx = wmax[0];
    for (int w = 1; w < 4; ++w) mx = wmax[w] > mx ? wmax[w] : mx;
    atomicMax(&a.maxkey[u], mx);
  }
  for (int i = tid; i < kBins; i += 256) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&a.hist1[(size_t)u * kBins + i], c);
  }
}

// Clears the per-unit histograms and maxima.
__global__ __launch_bounds__(256) void init_kernel(uint32_t* hist1, uint32_t* hist2,
                                                   uint32_t* maxkey) {
  const int u = blockIdx.x;
  for (int i = threadIdx.x; i < kBins; i += 256) {
    hist1[(size_t)u * kBins + i] = 0u;
    hist2[(size_t)u * kBins + i] = 0u;
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
  const int b = u / a.Hkv;
  const int L = clamp_len(a.seq_lens[b], a.max_seq_len);
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

int indexer_tokens_per_iteration(int pair_count) { return 4 * (kWave / (pair_count / 4)) * 8; }
int indexer_max_tokens_per_wg() { return kMaxTileTokens; }

hipError_t launch_init(uint32_t* hist1, uint32_t* hist2, uint32_t* maxkey, int units,
                       hipStream_t stream) {
  init_kernel<<<units, 256, 0, stream>>>(hist1, hist2, maxkey);
  return hipGetLastError();
}

hipError_t launch_indexer(const IndexArgs& a, int units, hipStream_t stream) {
  const int tiles = (a.max_seq_len + a.tokens_per_wg - 1) / a.tokens_per_wg;
  dim3 grid(tiles, units);
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

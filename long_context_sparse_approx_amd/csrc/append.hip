// Appending the new tokens' keys and values to the paged cache, in either key
// layout: whole keys, or split keys -- the scored RoPE pairs in one array and
// the other dims in another ("FASA: Frequency-aware Sparse Attention",
// section 3, variants: FASA-M keeps only the dominant key components
// resident and moves the remaining key components and the values elsewhere).
//
// A pure copy, bound by HBM: 2 * d * 2 bytes read and written per token and
// kv head.  One workgroup takes kAppendTokens consecutive new tokens; thread
// (h, slice) moves the 16-byte slice of every one of them, all loads issued
// before the stores.
#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

namespace {

constexpr int kAppendTokens = 4;

template <int D>
__global__ __launch_bounds__(1024) void append_kernel(AppendArgs a) {
  constexpr int S = D / 8;  // 16-byte slices per row
  const int tid = threadIdx.x;
  if (tid >= a.Hkv * S) return;
  const int h = tid / S;
  const int dim = (tid - h * S) * 8;
  const int lo = 2 * a.pair_begin;
  const int nd = 2 * a.pair_count;
  // Destination of this thread's key slice: the whole-key row, or the
  // scored-dims row, or the rest row.
  uint16_t* kdst;
  int kld;
  if (!a.k_rest) {
    kdst = a.k_cache + dim;
    kld = D;
  } else if (dim >= lo && dim < lo + nd) {
    kdst = a.k_cache + (dim - lo);
    kld = nd;
  } else {
    kdst = a.k_rest + (dim < lo ? dim : dim - nd);
    kld = D - nd;
  }
  const int64_t ntok = (int64_t)a.B * a.T;
  const int64_t tok0 = (int64_t)blockIdx.x * kAppendTokens;
  uint4 kv[kAppendTokens], vv[kAppendTokens];
  int64_t row[kAppendTokens];
#pragma unroll
  for (int i = 0; i < kAppendTokens; ++i) {
    const int64_t tok = tok0 + i;  // b * T + t
    row[i] = -1;
    if (tok < ntok) {
      const int b = (int)(tok / a.T);
      const int t = (int)(tok - (int64_t)b * a.T);
      const int pos = clamp_len(a.seq_lens[b], a.max_seq_len) - a.T + t;
      if (pos >= 0) {  // tokens before the start of the sequence are skipped
        int blk = a.block_table[(size_t)b * a.max_blocks + (pos >> 4)];
        blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
        row[i] = ((int64_t)blk * a.Hkv + h) * kBlockTokens + (pos & 15);
        const size_t src = ((size_t)tok * a.Hkv + h) * D + dim;
        kv[i] = *reinterpret_cast<const uint4*>(a.k_new + src);
        vv[i] = *reinterpret_cast<const uint4*>(a.v_new + src);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kAppendTokens; ++i) {
    if (row[i] >= 0) {
      *reinterpret_cast<uint4*>(kdst + (size_t)row[i] * kld) = kv[i];
      *reinterpret_cast<uint4*>(a.v_cache + (size_t)row[i] * D + dim) = vv[i];
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t ntok = (int64_t)a.B * a.T;
  if (ntok == 0) return hipSuccess;
  const int64_t grid = (ntok + kAppendTokens - 1) / kAppendTokens;
  const int threads = (a.Hkv * (a.d / 8) + 63) / 64 * 64;
  if (grid > 0x7fffffff || threads > 1024) return hipErrorInvalidValue;
  if (a.d == 128)
    append_kernel<128><<<(unsigned)grid, threads, 0, stream>>>(a);
  else if (a.d == 64)
    append_kernel<64><<<(unsigned)grid, threads, 0, stream>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ssa

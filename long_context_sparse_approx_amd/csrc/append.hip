// Appending the new tokens' keys and values to the paged cache, in either key
// layout: whole keys, or split keys -- the scored RoPE pairs in one array and
// the other dims in another ("FASA: Frequency-aware Sparse Attention",
// section 3, variants: FASA-M keeps only the dominant key components
// resident and moves the remaining key components and the values elsewhere).
//
// A pure copy, bound by HBM: 2 * d * 2 bytes read and written per token and
// kv head.  Thread (h, slice) of a workgroup moves the 16-byte slice of
// kAppendTokens consecutive new tokens per iteration.  A token's cache row is
// the same for the whole workgroup, so a few lanes of each wave resolve the
// positions (seq_lens) and blocks (block table) of the iteration's tokens
// with one load each, around the source loads (non-temporal, read once),
// and broadcast them.  Workgroups stride over the token groups.
#include "ssa_device.h"
#include "ssa_launch.h"

namespace ssa {

namespace {

constexpr int kAppendTokens = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_once(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int D>
__global__ __launch_bounds__(1024) void append_kernel(AppendArgs a) {
  constexpr int S = D / 8;  // 16-byte slices per row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const bool active = tid < a.Hkv * S;
  const int h = active ? tid / S : 0;  // inactive threads load row 0 and store nothing
  const int dim = active ? (tid - h * S) * 8 : 0;
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
  const uint32_t ntok = (uint32_t)a.B * (uint32_t)a.T;  // < 2^31 (checked by the host)
  const uint32_t T = (uint32_t)a.T;
  const size_t src_ld = (size_t)a.Hkv * D;
  const uint16_t* ksrc = a.k_new + (size_t)h * D + dim;
  const uint16_t* vsrc = a.v_new + (size_t)h * D + dim;
  for (uint32_t tok0 = blockIdx.x * kAppendTokens; tok0 < ntok;
       tok0 += gridDim.x * kAppendTokens) {
    // Lane i < kAppendTokens of every wave resolves token tok0 + i: its
    // position (-1: none) and cache block; every lane takes them by shuffle.
    // Loads are unconditional (addresses clamped to the last token) so that
    // they all stay in flight together; only the stores are predicated.
    const uint32_t last = ntok - 1;
    const uint32_t tok_l = min(tok0 + (uint32_t)(lane & (kAppendTokens - 1)), last);
    const uint32_t b_l = tok_l / T;
    const int len_l = a.seq_lens[b_l];
    u32x4 kv[kAppendTokens], vv[kAppendTokens];
#pragma unroll
    for (int i = 0; i < kAppendTokens; ++i) {
      const uint32_t tok = min(tok0 + i, last);  // b * T + t
      kv[i] = load_once(ksrc + tok * src_ld);
      vv[i] = load_once(vsrc + tok * src_ld);
    }
    int pos_l = clamp_len(len_l, a.max_seq_len) - a.T + (int)(tok_l - b_l * T);
    if (tok0 + (uint32_t)(lane & (kAppendTokens - 1)) > last) pos_l = -1;
    // tokens before the start of the sequence have no position (-1)
    int blk_l = a.block_table[(size_t)b_l * a.max_blocks + (pos_l < 0 ? 0 : pos_l >> 4)];
    blk_l = blk_l < 0 ? 0 : (blk_l >= a.num_blocks ? a.num_blocks - 1 : blk_l);
#pragma unroll
    for (int i = 0; i < kAppendTokens; ++i) {
      const int pos = __shfl(pos_l, i);
      const int blk = __shfl(blk_l, i);
      if (active && pos >= 0) {
        const size_t row = ((size_t)blk * a.Hkv + h) * kBlockTokens + (pos & 15);
        *reinterpret_cast<u32x4*>(kdst + row * kld) = kv[i];
        *reinterpret_cast<u32x4*>(a.v_cache + row * D + dim) = vv[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t ntok = (int64_t)a.B * a.T;
  if (ntok == 0) return hipSuccess;
  const int threads = (a.Hkv * (a.d / 8) + 63) / 64 * 64;
  if (ntok > 0x7fffffff || threads > 1024) return hipErrorInvalidValue;
  // Enough workgroups to fill the device several times over; they stride.
  int64_t grid = (ntok + kAppendTokens - 1) / kAppendTokens;
  if (grid > 65536) grid = 65536;
  if (a.d == 128)
    append_kernel<128><<<(unsigned)grid, threads, 0, stream>>>(a);
  else if (a.d == 64)
    append_kernel<64><<<(unsigned)grid, threads, 0, stream>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ssa

// Measurement aids: the HBM read rate this device delivers for the two
// access patterns of the decode step's bandwidth-bound kernels -- a long
// contiguous read (the indexer streams every cached key's scored dims) and a
// gather of scattered fixed-size rows (the attention reads the selected
// tokens' K and V rows through the block table).  Timing these beside the
// step says how far each kernel is from what the memory system gives for
// its pattern, which the published peak does not.
//
// Both kernels fold every 32-bit word they read by XOR into the sink word of
// their workgroup (a wave reduction, then one integer atomic per wave into
// slot blockIdx.x mod SSA_MEASURE_SINK_WORDS, so no address is contended), so
// the loads cannot be dropped and the XOR of the sink words does not depend
// on the order of the work.
#include <hip/hip_runtime.h>

#include "ssa.h"

namespace ssa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__device__ __forceinline__ void wave_xor_to(uint32_t v, uint32_t* sink) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off);
  if ((threadIdx.x & 63) == 0 && v) atomicXor(&sink[blockIdx.x % SSA_MEASURE_SINK_WORDS], v);
}

constexpr int kMT = 256;         // threads per workgroup
constexpr int kStreamWG = 2048;  // workgroups of the stream

// n16 16-byte words of src, grid-stride, non-temporal loads: a wave's loads
// cover 1 KiB of consecutive memory and consecutive waves the next ones.
// The fastest of a sweep over 1024-4096 workgroups, 1 or 4 loads in flight
// per thread, plain or non-temporal loads, and one contiguous range per
// workgroup (1 GiB in 152-155 us).
__global__ __launch_bounds__(kMT) void stream_kernel(const u32x4* __restrict__ src, size_t n16,
                                                     uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kMT;
  uint32_t acc = 0u;
  for (size_t i = (size_t)blockIdx.x * kMT + threadIdx.x; i < n16; i += stride)
    acc ^= fold(__builtin_nontemporal_load(src + i));
  wave_xor_to(acc, sink);
}

// n rows of LPR 16-byte words each (row r at src + r * LPR words); a wave
// reads 64 / LPR rows per load instruction, kGatherUnroll instructions in
// flight.  Row ids are clamped into [0, num_rows).
constexpr int kGatherUnroll = 8;
template <int LPR>
__global__ __launch_bounds__(kMT) void gather_kernel(const u32x4* __restrict__ src,
                                                     int64_t num_rows,
                                                     const int32_t* __restrict__ rows, int64_t n,
                                                     uint32_t* sink) {
  constexpr int RPI = 64 / LPR;  // rows per load instruction
  constexpr int RPW = RPI * kGatherUnroll;  // rows per wave per round
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kMT + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kMT) >> 6;
  uint32_t acc = 0u;
  for (int64_t base = wave * RPW; base < n; base += nwaves * RPW) {
    u32x4 v[kGatherUnroll];
    bool ok[kGatherUnroll];
#pragma unroll
    for (int k = 0; k < kGatherUnroll; ++k) {
      const int64_t i = base + k * RPI + lane / LPR;
      ok[k] = i < n;
      const int64_t r = rows[ok[k] ? i : n - 1];
      const int64_t rc = r < 0 ? 0 : (r >= num_rows ? num_rows - 1 : r);
      v[k] = src[rc * LPR + (lane % LPR)];
    }
#pragma unroll
    for (int k = 0; k < kGatherUnroll; ++k) acc ^= ok[k] ? fold(v[k]) : 0u;
  }
  wave_xor_to(acc, sink);
}

}  // namespace

}  // namespace ssa

extern "C" int ssa_measure_stream(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return SSA_ERR_INVALID;
  const size_t n16 = bytes / 16;
  size_t wg = (n16 + ssa::kMT - 1) / ssa::kMT;
  wg = wg < (size_t)ssa::kStreamWG ? wg : (size_t)ssa::kStreamWG;
  ssa::stream_kernel<<<(unsigned)wg, ssa::kMT, 0, (hipStream_t)stream>>>(
      static_cast<const ssa::u32x4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? SSA_OK : SSA_ERR_HIP;
}

extern "C" int ssa_measure_gather(const void* src, size_t row_bytes, int64_t num_rows,
                                  const int32_t* rows, int64_t n, uint32_t* sink, void* stream) {
  if (!src || !sink || !rows || num_rows < 1 || n < 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return SSA_ERR_INVALID;
  if (row_bytes < 16 || row_bytes > 1024 || (row_bytes & (row_bytes - 1)) != 0)
    return SSA_ERR_INVALID;
  if (n == 0) return SSA_OK;
  const hipStream_t s = (hipStream_t)stream;
  const ssa::u32x4* s4 = static_cast<const ssa::u32x4*>(src);
  // workgroups: enough for every row once, at most 4096
  const int64_t rows_per_wg_round = (int64_t)(ssa::kMT / 64) * 64 * ssa::kGatherUnroll;
  auto grid = [&](int lpr) {
    const int64_t per = rows_per_wg_round / lpr;
    const int64_t wg = (n + per - 1) / per;
    return (unsigned)(wg < 4096 ? wg : 4096);
  };
  switch (row_bytes) {
    case 16: ssa::gather_kernel<1><<<grid(1), ssa::kMT, 0, s>>>(s4, num_rows, rows, n, sink); break;
    case 32: ssa::gather_kernel<2><<<grid(2), ssa::kMT, 0, s>>>(s4, num_rows, rows, n, sink); break;
    case 64: ssa::gather_kernel<4><<<grid(4), ssa::kMT, 0, s>>>(s4, num_rows, rows, n, sink); break;
    case 128: ssa::gather_kernel<8><<<grid(8), ssa::kMT, 0, s>>>(s4, num_rows, rows, n, sink); break;
    case 256: ssa::gather_kernel<16><<<grid(16), ssa::kMT, 0, s>>>(s4, num_rows, rows, n, sink); break;
    case 512: ssa::gather_kernel<32><<<grid(32), ssa::kMT, 0, s>>>(s4, num_rows, rows, n, sink); break;
    case 1024: ssa::gather_kernel<64><<<grid(64), ssa::kMT, 0, s>>>(s4, num_rows, rows, n, sink); break;
    default: return SSA_ERR_INVALID;
  }
  return hipGetLastError() == hipSuccess ? SSA_OK : SSA_ERR_HIP;
}

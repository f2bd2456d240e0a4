// ring_rows.hip -- copy fp32 [kv, score] state rows into their ring slots,
// for gfx950.
//
// What is copied follows the DeepSeek-V4.1 insert page ("vllm.models.
// deepseek_v41.common.ops.fused_compress_quant_cache": `save_ring_rows`, and
// the ring rule in the `fused_save_compress_norm` docstring): row i goes to
// the ring slot s = slot_mapping[i] = block * capacity + (position % capacity),
// i.e. to state + (s / capacity) * state_stride + (s % capacity) *
// state_row_stride; slot -1 is skipped (and, by our reading, any negative slot
// or one past the last ring row).  The copy is bit-for-bit.
//
// One wave per row: lane l moves 16 bytes per 256-value chunk through raw
// buffer loads/stores whose range is the row (or empty for a skipped row, so
// the hardware drops the accesses without a branch).  Rows stay cached (plain
// stores): the ring is read back by the next chunk of the same request.
#include "kernels.hpp"

namespace mxs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWave = 2;
constexpr int kWavesPerBlock = 4;

template <int kChunks>  // width / 256 when known, else 0 (generic loop)
__global__ __launch_bounds__(kWave * kWavesPerBlock) void ring_rows_kernel(const RingArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t first = ((int64_t)xcd_contiguous_block() * kWavesPerBlock + wave) * kRowsPerWave;
  const uint32_t row_bytes = (uint32_t)(a.width * 4);

  __amdgpu_buffer_rsrc_t src[kRowsPerWave], dst[kRowsPerWave];
#pragma unroll
  for (int p = 0; p < kRowsPerWave; ++p) {
    const int64_t i = first + p;
    const int64_t s = i < a.num_rows ? a.slots[i] : -1;
    const bool ok = s >= 0 && s < (int64_t)a.num_slots;
    const uint32_t blk = ok ? (uint32_t)s / a.capacity : 0u;
    const uint32_t r = ok ? (uint32_t)s - blk * a.capacity : 0u;
    src[p] = buffer_at(a.rows + (ok ? i * a.row_stride : 0), ok ? row_bytes : 0u);
    dst[p] = buffer_at(a.state + (int64_t)blk * a.state_stride + (int64_t)r * a.state_row_stride,
                       ok ? row_bytes : 0u);
  }
  if constexpr (kChunks > 0) {
    u32x4 v[kRowsPerWave][kChunks];
#pragma unroll
    for (int p = 0; p < kRowsPerWave; ++p)
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
        v[p][c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(src[p], (c * 64 + lane) * 16, 0, 0));
#pragma unroll
    for (int p = 0; p < kRowsPerWave; ++p)
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
        __builtin_amdgcn_raw_buffer_store_b128(v[p][c], dst[p], (c * 64 + lane) * 16, 0, 0);
  } else {
    for (uint32_t off = lane * 16u; off < row_bytes; off += 64u * 16u) {
#pragma unroll
      for (int p = 0; p < kRowsPerWave; ++p) {
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src[p], off, 0, 0));
        __builtin_amdgcn_raw_buffer_store_b128(v, dst[p], off, 0, 0);
      }
    }
  }
}

}  // namespace

hipError_t launch_ring_rows(const RingArgs& a, hipStream_t stream) {
  constexpr int64_t kPerBlock = (int64_t)kWavesPerBlock * kRowsPerWave;
  const int64_t blocks = (a.num_rows + kPerBlock - 1) / kPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (a.width == 1024)
    hipLaunchKernelGGL(ring_rows_kernel<4>, dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(ring_rows_kernel<0>, dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace mxs

// bench_probes.hip -- memory-system probes for the benchmark (libmxprobe.so).
//
// Plain kernels with the memory traffic of the MXFP4 store and none of its
// arithmetic, used by bench.py --probes to measure what the HBM of one
// MI355X delivers for each access pattern the store path makes:
//   probe_read       sequential non-temporal reads (16 B per lane, 64 B per thread)
//   probe_write      sequential writes: plain, or written through (NT + SC1)
//   probe_copy_rows  per row: read a 1 KiB row, write a 272-byte row derived
//                    from it, four rows per wave assembled in LDS and written
//                    as 16-byte chunks -- the store's traffic and write form.
//                    With `order`, output row s comes from input row order[s]
//                    (a gather in output order, as the slot-order store does);
//                    without, row t goes to row t (both sides sequential).
//                    Its 16-byte stores are plain or written through (NT + SC1).
//   probe_copy_wide  per row: copy a row of `width` bytes (a multiple of 1 KiB)
//                    to output row order[t] (or t), one wave per row -- the
//                    ring-state save's traffic.
//   probe_copy_expand  rows in order: read `in_bytes`, write `out_bytes` derived
//                    from them, one wave per row, 16 B per lane -- the traffic of
//                    the gather-dequant (272 -> 1024, non-temporal stores) and of
//                    the compress-ratio-1 norm (2048 -> 1024, written through).
//   probe_scatter_dwords  dst[idx[t]] = t for t < n (idx int64, in range):
//                    scattered 4-byte writes, 1-8 per thread -- the inverse
//                    map's traffic.
//   probe_lds        LDS and matrix-core rates of one CU (1024-thread
//                    workgroups holding 96 KB of LDS, one per CU): contiguous
//                    ds_read_b128, ds_read_b64_tr_b16, ds_write_b128,
//                    ds_write_b64, or 16x16x32 bf16 MFMAs alone -- the
//                    budget a kernel that stages operands in LDS works with.
//   probe_lds_pattern  one ds_read_b128 / ds_write_b128 per lane at a given
//                    lane -> 16-byte-unit map, repeated: the bank conflicts
//                    of an access pattern (rocprofv3 SQ_LDS_BANK_CONFLICT).
//   probe_empty      an empty kernel: the launch floor of a given grid.
// The written bytes depend on the loaded ones so no load can be dropped; a
// read-only probe writes one dword only when its checksum hits a constant.
// Not part of the library's product path.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBufNT = 2;
constexpr int kBufNTDevice = kBufNT | 16;  // NT + SC1: written through to memory
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_at(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}

// Consecutive logical blocks on one XCD (workgroups go round-robin over the 8).
__device__ __forceinline__ uint32_t xcd_contiguous_block() {
  const uint32_t nb = gridDim.x, full = nb & ~7u, b = blockIdx.x;
  return b < full ? (b & 7u) * (full >> 3) + (b >> 3) : b;
}

// 256 threads, each reading four 16-byte vectors, 16 KiB per block.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src,
                                                         uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)xcd_contiguous_block() * 1024 + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(src + base + j * 256);
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

template <int kPol>
__global__ __launch_bounds__(256) void probe_write_kernel(u32x4* __restrict__ dst) {
  const int64_t block = xcd_contiguous_block();
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = u32x4{t, t ^ 1u, t ^ 2u, (uint32_t)j};
    if constexpr (kPol == 0)
      dst[block * 1024 + t + j * 256] = v;
    else
      __builtin_amdgcn_raw_buffer_store_b128(v, buffer_at(dst + block * 1024, 16384), (t + j * 256) * 16, 0, kPol);
  }
}

constexpr int kRowsPerWave = 4;
constexpr int kWavesPerBlock = 4;
constexpr int kOut = 272;                    // bytes per output row
constexpr int kSpan = kRowsPerWave * kOut;   // 1088 bytes per wave

template <int kPol>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void probe_copy_rows_kernel(
    const uint8_t* __restrict__ src, int64_t rows, const int32_t* __restrict__ order,
    uint8_t* __restrict__ dst) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = ((int64_t)xcd_contiguous_block() * kWavesPerBlock + wave) * kRowsPerWave;
  if (r0 >= rows) return;
  int32_t tok[kRowsPerWave];
#pragma unroll
  for (int p = 0; p < kRowsPerWave; ++p) tok[p] = order ? order[r0 + p] : (int32_t)(r0 + p);
  u32x4 v[kRowsPerWave];
#pragma unroll
  for (int p = 0; p < kRowsPerWave; ++p) {
    const bool ok = tok[p] >= 0;
    const __amdgpu_buffer_rsrc_t rs = buffer_at(src + (ok ? (int64_t)tok[p] * 1024 : 0), ok ? 1024u : 0u);
    v[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, 0, kBufNT));
  }
  __shared__ uint32_t stage[kWavesPerBlock][kSpan / 4];
  uint32_t* st = stage[wave];
  uint32_t valid = 0;
#pragma unroll
  for (int p = 0; p < kRowsPerWave; ++p) {
    valid |= (tok[p] >= 0 ? 1u : 0u) << p;
    const uint32_t x = v[p].x ^ v[p].y ^ v[p].z ^ v[p].w;
    st[p * (kOut / 4) + lane] = x;
    if ((lane & 15) == 12) st[p * (kOut / 4) + 64 + (lane >> 4)] = x ^ 0x5A5A5A5Au;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const __amdgpu_buffer_rsrc_t rs = buffer_at(dst + r0 * kOut, (uint32_t)kSpan);
#pragma unroll
  for (int c0 = 0; c0 < kSpan / 16; c0 += kWave) {
    const int c = c0 + lane;
    if (c < kSpan / 16) {
      const u32x4 d = *reinterpret_cast<const u32x4*>(&st[4 * c]);
      const uint32_t off = (valid >> (c / (kOut / 16))) & 1u ? (uint32_t)(16 * c) : 0x7FFFFFF0u;
      __builtin_amdgcn_raw_buffer_store_b128(d, rs, off, 0, kPol);
    }
  }
}

// One wave per row; lane l moves bytes 16l + 1024j of it.
__global__ __launch_bounds__(256) void probe_copy_wide_kernel(const u32x4* __restrict__ src, int64_t rows,
                                                              int64_t width16, const int64_t* __restrict__ order,
                                                              u32x4* __restrict__ dst) {
  const int64_t t = (int64_t)xcd_contiguous_block() * 4 + (threadIdx.x >> 6);
  if (t >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t d = order ? order[t] : t;
  for (int64_t j = lane; j < width16; j += 64) dst[d * width16 + j] = src[t * width16 + j];
}

// A wave moves kRows consecutive rows (one span of kRows * kIn bytes in, one
// of kRows * kOut bytes out), four waves per block.  Lanes load 16-byte
// chunks of the input span (lanes past its chunks reload one, which the
// caches serve) and write 16-byte chunks of the output span that depend on
// them.  A last, partial span is cut by the buffer ranges.
template <int kIn, int kOut, int kPol, int kRows>
__global__ __launch_bounds__(256) void probe_copy_expand_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                                uint8_t* __restrict__ dst) {
  static_assert(kIn % 16 == 0 && (kRows * kOut) % 1024 == 0, "16-byte chunks, 1 KiB output steps");
  constexpr int kInChunks = kRows * kIn / 16;
  const int64_t r0 = ((int64_t)xcd_contiguous_block() * 4 + (threadIdx.x >> 6)) * kRows;
  if (r0 >= rows) return;
  const int64_t nr = rows - r0 < kRows ? rows - r0 : kRows;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t in = buffer_at(src + r0 * kIn, (uint32_t)(nr * kIn));
  u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < (kInChunks + 63) / 64; ++i) {
    const int c = (i * 64 + lane) % kInChunks;
    v ^= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(in, c * 16, 0, 0));
  }
  const __amdgpu_buffer_rsrc_t out = buffer_at(dst + r0 * kOut, (uint32_t)(nr * kOut));
#pragma unroll
  for (int j = 0; j < kRows * kOut / 1024; ++j)
    __builtin_amdgcn_raw_buffer_store_b128(v ^ u32x4{(uint32_t)j, 0u, 0u, 0u}, out, (j * 64 + lane) * 16, 0, kPol);
}

// Each thread writes kPer entries: its indices are loaded first, then the
// scattered dwords are stored.
template <int kPer>
__global__ __launch_bounds__(256) void probe_scatter_dwords_kernel(const int64_t* __restrict__ idx, int64_t n,
                                                                   int32_t* __restrict__ dst) {
  const int64_t t0 = ((int64_t)blockIdx.x * 256) * kPer + threadIdx.x;
  int64_t s[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) s[j] = t0 + j * 256 < n ? idx[t0 + j * 256] : -1;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (s[j] >= 0) dst[s[j]] = (int32_t)(t0 + j * 256);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// kind 0: ds_read_b128, 1: ds_read_b64_tr_b16, 2: ds_write_b128,
// 3: ds_write_b64 (each wave instruction on 1 KB / 512 B of contiguous
// LDS), 4: two independent 16x16x32 bf16 MFMAs per step.  The base offset
// passes through an empty asm each iteration, so no access is hoisted or
// merged.
template <int kKind>
__global__ __launch_bounds__(1024) void probe_lds_kernel(uint32_t* __restrict__ out, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[24576];  // 96 KB: one workgroup per CU
  for (int i = threadIdx.x; i < 24576; i += 1024) lds[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  char* base = reinterpret_cast<char*>(lds);
  u32x4 acc = {0u, 0u, 0u, 0u};
  f32x4 m[8];
  for (int j = 0; j < 8; ++j) m[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const bf16x8 qa = __builtin_bit_cast(bf16x8, u32x4{lane, 3u, 5u, 7u});
  for (int it = 0; it < iters; ++it) {
    uint32_t o = (uint32_t)it * 8192u;
    asm volatile("" : "+v"(o));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (kKind == 0) {
        acc ^= *reinterpret_cast<const u32x4*>(base + ((w * 4096u + lane * 16u + o + u * 1024u) & 0xFFF0u));
      } else if constexpr (kKind == 1) {
        const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(base + ((w * 4096u + lane * 8u + o + u * 512u) & 0xFFF8u)));
        acc[u & 3] ^= (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[3] << 16);
      } else if constexpr (kKind == 2) {
        *reinterpret_cast<u32x4*>(base + ((w * 4096u + lane * 16u + o + u * 1024u) & 0xFFF0u)) =
            u32x4{o, lane, w, (uint32_t)u};
      } else if constexpr (kKind == 3) {
        *reinterpret_cast<u32x2*>(base + ((w * 4096u + lane * 8u + o + u * 512u) & 0xFFF8u)) = u32x2{o, lane};
      } else {
        const bf16x8 kb = __builtin_bit_cast(bf16x8, u32x4{o ^ (uint32_t)u, lane, w, 1u});
        m[(2 * u) & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qa, m[(2 * u) & 7], 0, 0, 0);
        m[(2 * u + 1) & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kb, m[(2 * u + 1) & 7], 0, 0, 0);
      }
    }
  }
  if constexpr (kKind == 2 || kKind == 3) {
    __syncthreads();
    acc[0] = lds[threadIdx.x * 16];
  }
  float s = 0.0f;
  for (int j = 0; j < 8; ++j) s += m[j][0] + m[j][1] + m[j][2] + m[j][3];
  out[(size_t)blockIdx.x * 1024 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ __float_as_uint(s);
}

// LDS bank conflicts of one access pattern: one wave per workgroup, 64 KB
// of LDS; lane l reads or writes the 16-byte unit units[l] (0..4095) `iters`
// times (ds_read_b128 / ds_write_b128), its offset passing through an empty
// asm each time.  Run under rocprofv3's SQ_LDS_BANK_CONFLICT counter.
template <bool kWrite>
__global__ __launch_bounds__(64) void probe_lds_pattern_kernel(const uint32_t* __restrict__ units,
                                                               uint32_t* __restrict__ out, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[16384];
  const uint32_t lane = threadIdx.x;
  for (int i = lane; i < 16384; i += 64) lds[i] = (uint32_t)i;
  __syncthreads();
  uint32_t off = (units[lane] & 4095u) * 16u;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(off));
    if constexpr (kWrite)
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(lds) + off) = u32x4{(uint32_t)it, lane, 2u, 1u};
    else
      acc ^= *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(lds) + off);
  }
  __syncthreads();
  if constexpr (kWrite) acc[0] = lds[lane];
  out[(size_t)blockIdx.x * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(256) void probe_empty_kernel() {}

int status(hipError_t e) { return e == hipSuccess ? 0 : -7; }

template <int kIn, int kOut, int kPol>
int launch_expand(const uint8_t* s, int64_t rows, int rows_per_wave, uint8_t* d, hipStream_t stream) {
  const int64_t per_block = 4 * (int64_t)rows_per_wave;
  if ((rows + per_block - 1) / per_block > 0x7FFFFFFF) return -1;
  const dim3 grid((unsigned)((rows + per_block - 1) / per_block)), block(256);
  switch (rows_per_wave) {
    case 1: hipLaunchKernelGGL((probe_copy_expand_kernel<kIn, kOut, kPol, 1>), grid, block, 0, stream, s, rows, d); break;
    case 2: hipLaunchKernelGGL((probe_copy_expand_kernel<kIn, kOut, kPol, 2>), grid, block, 0, stream, s, rows, d); break;
    case 4: hipLaunchKernelGGL((probe_copy_expand_kernel<kIn, kOut, kPol, 4>), grid, block, 0, stream, s, rows, d); break;
    case 8: hipLaunchKernelGGL((probe_copy_expand_kernel<kIn, kOut, kPol, 8>), grid, block, 0, stream, s, rows, d); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16 KiB) from src.  sink: one device dword.
int probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16384 || bytes / 16384 > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)(bytes / 16384)), dim3(256), 0,
                     (hipStream_t)stream, static_cast<const u32x4*>(src), sink);
  return status(hipGetLastError());
}

// Writes `bytes` (a multiple of 16 KiB) to dst; through != 0: NT + SC1 stores.
int probe_write(void* dst, int64_t bytes, int through, void* stream) {
  if (!dst || bytes <= 0 || bytes % 16384 || bytes / 16384 > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(through ? probe_write_kernel<kBufNTDevice> : probe_write_kernel<0>,
                     dim3((unsigned)(bytes / 16384)), dim3(256), 0, (hipStream_t)stream,
                     static_cast<u32x4*>(dst));
  return status(hipGetLastError());
}

// rows (a multiple of 16) output rows of 272 bytes in dst, each from a
// 1 KiB row of src: row order[s] (entries in [0, src rows) or -1: row not
// written) or, with order NULL, row s.  src and dst 16-byte aligned.
// through != 0: NT + SC1 stores.
int probe_copy_rows(const void* src, int64_t rows, const int32_t* order, void* dst, int through,
                    void* stream) {
  if (!src || !dst || rows <= 0 || rows % 16 || rows / 16 > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(through ? probe_copy_rows_kernel<kBufNTDevice> : probe_copy_rows_kernel<0>,
                     dim3((unsigned)(rows / 16)), dim3(kWave * kWavesPerBlock), 0, (hipStream_t)stream, static_cast<const uint8_t*>(src), rows, order,
                     static_cast<uint8_t*>(dst));
  return status(hipGetLastError());
}

// rows rows of `width` bytes (a multiple of 1024) from src to dst row
// order[t] (entries in [0, rows), a permutation) or, with order NULL, row t.
// src and dst 16-byte aligned.
int probe_copy_wide(const void* src, int64_t rows, int64_t width, const int64_t* order, void* dst,
                    void* stream) {
  if (!src || !dst || rows <= 0 || width <= 0 || width % 1024 || (rows + 3) / 4 > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(probe_copy_wide_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     (hipStream_t)stream, static_cast<const u32x4*>(src), rows, width / 16, order,
                     static_cast<u32x4*>(dst));
  return status(hipGetLastError());
}

// rows rows of in_bytes in src, in order, to rows of out_bytes in dst, with
// rows_per_wave in {1, 2, 4, 8}: (in_bytes, out_bytes, policy) = (272, 1024,
// 2) (non-temporal stores) or (2048, 1024, 18) (stores written through);
// anything else is refused.
int probe_copy_expand(const void* src, int64_t rows, int in_bytes, int out_bytes, int policy, int rows_per_wave,
                      void* dst, void* stream) {
  if (!src || !dst || rows <= 0) return -1;
  const auto s = static_cast<const uint8_t*>(src);
  const auto d = static_cast<uint8_t*>(dst);
  if (in_bytes == 272 && out_bytes == 1024 && policy == kBufNT)
    return launch_expand<272, 1024, kBufNT>(s, rows, rows_per_wave, d, (hipStream_t)stream);
  if (in_bytes == 2048 && out_bytes == 1024 && policy == kBufNTDevice)
    return launch_expand<2048, 1024, kBufNTDevice>(s, rows, rows_per_wave, d, (hipStream_t)stream);
  return -1;
}

// dst[idx[t]] = t for t < n, per_thread in {1, 2, 4, 8}.  Every idx[t] must
// lie in [0, dst_len) or be negative (skipped); checked by the caller, as the
// kernel writes where the entries say.
int probe_scatter_dwords(const int64_t* idx, int64_t n, int per_thread, int32_t* dst, void* stream) {
  if (!idx || !dst || n <= 0) return -1;
  const int64_t per_block = 256 * (int64_t)per_thread;
  const int64_t blocks = (n + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return -1;
  const dim3 grid((unsigned)blocks), block(256);
  switch (per_thread) {
    case 1: hipLaunchKernelGGL(probe_scatter_dwords_kernel<1>, grid, block, 0, (hipStream_t)stream, idx, n, dst); break;
    case 2: hipLaunchKernelGGL(probe_scatter_dwords_kernel<2>, grid, block, 0, (hipStream_t)stream, idx, n, dst); break;
    case 4: hipLaunchKernelGGL(probe_scatter_dwords_kernel<4>, grid, block, 0, (hipStream_t)stream, idx, n, dst); break;
    case 8: hipLaunchKernelGGL(probe_scatter_dwords_kernel<8>, grid, block, 0, (hipStream_t)stream, idx, n, dst); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

// LDS / MFMA rate probe: `blocks` workgroups of 1024 threads, `iters`
// iterations of 8 accesses (kinds 0-3) or 16 MFMAs (kind 4) per wave;
// `out` holds blocks * 1024 dwords.
int probe_lds(int kind, int64_t blocks, int iters, uint32_t* out, void* stream) {
  if (!out || blocks <= 0 || blocks > 0x7FFFFFFF || iters <= 0) return -1;
  const dim3 grid((unsigned)blocks), block(1024);
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_lds_kernel<0>, grid, block, 0, (hipStream_t)stream, out, iters); break;
    case 1: hipLaunchKernelGGL(probe_lds_kernel<1>, grid, block, 0, (hipStream_t)stream, out, iters); break;
    case 2: hipLaunchKernelGGL(probe_lds_kernel<2>, grid, block, 0, (hipStream_t)stream, out, iters); break;
    case 3: hipLaunchKernelGGL(probe_lds_kernel<3>, grid, block, 0, (hipStream_t)stream, out, iters); break;
    case 4: hipLaunchKernelGGL(probe_lds_kernel<4>, grid, block, 0, (hipStream_t)stream, out, iters); break;
    default: return -1;
  }
  return status(hipGetLastError());
}

// LDS access-pattern probe: `blocks` one-wave workgroups, each lane l
// repeating a 16-byte read (write == 0) or write at unit units[l] (a device
// array of 64 entries in [0, 4096)) `iters` times; `out` holds blocks * 64
// dwords.
int probe_lds_pattern(const uint32_t* units, int write, int64_t blocks, int iters, uint32_t* out, void* stream) {
  if (!units || !out || blocks <= 0 || blocks > 0x7FFFFFFF || iters <= 0) return -1;
  const dim3 grid((unsigned)blocks), block(64);
  if (write)
    hipLaunchKernelGGL(probe_lds_pattern_kernel<true>, grid, block, 0, (hipStream_t)stream, units, out, iters);
  else
    hipLaunchKernelGGL(probe_lds_pattern_kernel<false>, grid, block, 0, (hipStream_t)stream, units, out, iters);
  return status(hipGetLastError());
}

// An empty kernel over `blocks` workgroups of 256 threads.
int probe_empty(int64_t blocks, void* stream) {
  if (blocks <= 0 || blocks > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(probe_empty_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream);
  return status(hipGetLastError());
}

}  // extern "C"

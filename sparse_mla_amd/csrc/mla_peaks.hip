// Attainable-peak microbenchmarks (streaming HBM read, random 1152-byte row
// gather by LDS-DMA, dense bf16 MFMA) behind the C ABI of mla_peaks.h.  They
// price the decode against what this chip attains, beside the published peaks;
// none of them computes anything of the method.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_peaks.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRowBytes = 1152;     // 576 bf16 values per cached position
constexpr int kBlkRows = 32;        // rows per gathered block
constexpr int kBlkBytes = kBlkRows * kRowBytes;
constexpr int kNbuf = 4;
constexpr int kMaxRowsPerWg = 1024;

__device__ __forceinline__ i32x4 raw_buffer(const void* base, uint32_t num_records) {
  const uint64_t addr = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
  r[3] = 0x00020000;  // raw buffer, 32-bit data format
  return r;
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds_base + 16 lane;
// offsets at or past num_records read zeros without touching memory.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Grid-stride 16-byte loads, eight in flight per lane.
__global__ __launch_bounds__(256) void stream_kernel(const uint4* p, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].w;
  }
  for (; i < n16; i += stride) acc ^= p[i].x;
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// The decode's gather: the row list is staged in LDS first (a compiler-visible
// load inside the loop would get a wait that drains the gathers in flight),
// then block j goes out after block j - 3 has landed (barrier per block).
// Lane l of wave w moves 16 bytes of line m of row 8 w + l / 8 of the block.
__global__ __launch_bounds__(256, 1) void rows_kernel(const char* cache, uint32_t cache_bytes, const int32_t* rows,
                                                       int rows_per_wg, uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) char ring[kNbuf * kBlkBytes];
  __shared__ int srow[kMaxRowsPerWg];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t* mine = rows + (size_t)blockIdx.x * rows_per_wg;
  for (int i = tid; i < rows_per_wg; i += 256) srow[i] = mine[i];
  __syncthreads();
  const i32x4 rs = raw_buffer(cache, cache_bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;
  const int nblk = rows_per_wg / kBlkRows;
  const int key = 8 * wave + (lane >> 3);
  for (int j = 0; j < nblk + kNbuf - 1; ++j) {
    if (j >= kNbuf - 1) {
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");  // block j - 3 landed
      __syncthreads();
    }
    if (j < nblk) {
      const uint32_t off = (uint32_t)srow[j * kBlkRows + key] * (uint32_t)kRowBytes + 16u * (uint32_t)(lane & 7);
      const uint32_t dst = lds0 + (uint32_t)((j % kNbuf) * kBlkBytes) + (uint32_t)(8 * wave * 128);
#pragma unroll
      for (int m = 0; m < 9; ++m) lds_dma16(rs, dst + (uint32_t)(m * kBlkRows * 128), off + (uint32_t)(m * 128));
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (reinterpret_cast<const uint32_t*>(ring)[tid] == 0x9e3779b9u) sink[0] = 1u;
}

// 16 independent accumulators per wave, 16 MFMAs per round.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (float)(lane + k));
    b[k] = (__bf16)(0.002f * (float)(lane - k));
  }
  f32x16 acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m) s += acc[m][m];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : 2; }

}  // namespace

extern "C" int mlap_stream_read(const void* src, size_t bytes, int32_t num_wg, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0 || num_wg < 1)
    return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(stream_kernel, dim3(num_wg), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return launched();
}

extern "C" int mlap_row_gather(const void* cache, size_t cache_bytes, const int32_t* rows, int32_t num_wg,
                               int32_t rows_per_wg, uint32_t* sink, void* stream) {
  if (!cache || !rows || !sink || num_wg < 1 || rows_per_wg < kBlkRows || rows_per_wg > kMaxRowsPerWg ||
      rows_per_wg % kBlkRows != 0 || cache_bytes == 0 || cache_bytes > UINT32_MAX)
    return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(rows_kernel, dim3(num_wg), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const char*>(cache), (uint32_t)cache_bytes, rows, (int)rows_per_wg, sink);
  return launched();
}

extern "C" int mlap_mfma_bf16(int32_t num_wg, int32_t iters, float* sink, void* stream) {
  if (!sink || num_wg < 1 || iters < 1) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(mfma_kernel, dim3(num_wg), dim3(256), 0, static_cast<hipStream_t>(stream), (int)iters, sink);
  return launched();
}

// Measurement probes for the benchmark (libvbprobe.so; not part of the bound
// library): what the matrix cores and HBM sustain on the machine at hand,
// reported next to the published MI355X peaks.
//   vbp_mfma_loop  - fp32 MFMA blocks (v_mfma_f32_32x32x2f32) with four
//                    independent accumulator chains per wavefront, no memory
//                    traffic inside the loop; 4096 FLOP per block per wavefront.
//   vbp_read       - streams a buffer once (non-temporal 16-byte loads, four in
//                    flight per lane, one contiguous 16 KB segment per
//                    workgroup), one partial sum per workgroup written out.
//   vbp_write      - fills a buffer (16-byte non-temporal stores, same layout).
//   vbp_copy       - reads one buffer and writes another (same layout).
// Every entry point enqueues on the given stream and returns the launch status.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  float a = 1.0f + 1e-7f * lane;
  float b = 1.0f - 1e-7f * lane;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  // one value per workgroup keeps the chains live
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

constexpr int UNROLL = 4;
constexpr int SEG = 256 * UNROLL;  // float4 per workgroup: 16 KB, 4 KB per wavefront

// Each workgroup streams one contiguous 16 KB segment: wavefront w of it reads
// the 4 KB at w, with its UNROLL 16-byte loads (64 lanes x 16 B = 1 KB each)
// issued before any is used.  Short-lived workgroups over contiguous segments
// keep many DRAM pages streaming at once.
__device__ __forceinline__ long long seg_index(int u) {
  return (long long)blockIdx.x * SEG + (threadIdx.x >> 6) * (64 * UNROLL) + u * 64 + (threadIdx.x & 63);
}

__global__ __launch_bounds__(256) void read_kernel(const f32x4* __restrict__ p, long long n4, float* out) {
  f32x4 v[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const long long i = seg_index(u);
    v[u] = i < n4 ? __builtin_nontemporal_load(p + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) s += v[u].x + v[u].y + v[u].z + v[u].w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void write_kernel(f32x4* __restrict__ p, long long n4, float v) {
  const f32x4 x = {v, v, v, v};
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const long long i = seg_index(u);
    if (i < n4) __builtin_nontemporal_store(x, p + i);
  }
}

__global__ __launch_bounds__(256) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                   long long n4) {
  f32x4 v[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const long long i = seg_index(u);
    v[u] = i < n4 ? __builtin_nontemporal_load(src + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const long long i = seg_index(u);
    if (i < n4) __builtin_nontemporal_store(v[u], dst + i);
  }
}

long long stream_blocks(long long n4) { return (n4 + SEG - 1) / SEG; }

}  // namespace

extern "C" {

// blocks workgroups of 4 wavefronts, each running `iters` rounds of 4 MFMA blocks;
// out receives `blocks` floats.  FLOPs = blocks * 4 * iters * 4 * 4096.
int vbp_mfma_loop(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}

// Reads n floats (n a multiple of 4, p 16-byte aligned); out receives one float per
// workgroup (vbp_stream_blocks(n) of them).
int vbp_read(const float* p, long long n, float* out, void* stream) {
  if (!p || !out || n <= 0 || n % 4 || ((uintptr_t)p & 15)) return (int)hipErrorInvalidValue;
  if (stream_blocks(n / 4) > INT32_MAX) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)stream_blocks(n / 4)), dim3(256), 0, (hipStream_t)stream,
                     (const f32x4*)p, n / 4, out);
  return (int)hipGetLastError();
}

int vbp_write(float* p, long long n, float v, void* stream) {
  if (!p || n <= 0 || n % 4 || ((uintptr_t)p & 15)) return (int)hipErrorInvalidValue;
  if (stream_blocks(n / 4) > INT32_MAX) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(write_kernel, dim3((unsigned)stream_blocks(n / 4)), dim3(256), 0, (hipStream_t)stream, (f32x4*)p,
                     n / 4, v);
  return (int)hipGetLastError();
}

int vbp_copy(const float* src, float* dst, long long n, void* stream) {
  if (!src || !dst || n <= 0 || n % 4 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
    return (int)hipErrorInvalidValue;
  if (stream_blocks(n / 4) > INT32_MAX) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)stream_blocks(n / 4)), dim3(256), 0, (hipStream_t)stream,
                     (const f32x4*)src, (f32x4*)dst, n / 4);
  return (int)hipGetLastError();
}

long long vbp_stream_blocks(long long n) { return stream_blocks(n / 4); }

}  // extern "C"

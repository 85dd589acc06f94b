// Interval bound propagation (centre/radius form) through one Linear layer for
// a small batch, the case where the weight matrix is read from HBM once and
// dominates all traffic (the page's wide single-hidden-layer networks, Sec. 1;
// IBP as the cheap bound of Sec. 2.1).
//
// Output neurons run along the MFMA row dimension and the batch along its
// column dimension (v_mfma_f32_16x16x4f32, at most 16 inputs): each lane
// streams float4 pieces of its weight rows straight from HBM into registers
// (no LDS staging, nothing is reused), and the input centres / radii, which
// every wave reads, come from L2.  One chain of MFMAs accumulates W.c, a second
// |W|.r on the same weight registers.  Long rows are split over a grid
// dimension; partial sums then go to a workspace and a fixed-order finishing
// kernel adds them (one wavefront per output when there are many slices).
#include <hip/hip_runtime.h>

#include "vb_internal.h"

namespace vb {

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int NB = 8;          // MFMA blocks of 16 output neurons per wavefront
constexpr int ROWS = 16 * NB;  // output neurons per wavefront
constexpr int U = 2;           // 16-wide K steps whose loads are issued together

// float4 at a clamped element offset (always a valid address of the array)
__device__ __forceinline__ float4 ldg4(const float* __restrict__ p, long long off) {
  return *reinterpret_cast<const float4*>(p + off);
}

template <int AMODE>
__global__ __launch_bounds__(256) void ibp_narrow_kernel(NarrowIbp d) {
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * ROWS;
  if (n0 >= d.N) return;  // whole wavefront; the kernel has no barriers
  const int r16 = lane & 15, g = lane >> 4;
  const int kbeg = blockIdx.y * d.kchunk;
  const int kend = min(d.K, kbeg + d.kchunk);
  // A operand: lane (r16, g) holds weight row n0 + 16*blk + r16 and K index
  // 4*g + s of every 16-wide step s; B operand: input r16 at the same K index.
  const bool jok = r16 < d.batch;
  const long long xrow = (long long)(jok ? r16 : 0) * d.K;
  long long wrow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int n = n0 + 16 * b + r16;
    wrow[b] = (long long)(n < d.N ? n : d.N - 1) * d.K;
  }
  f32x4 ac[NB], ar[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    ac[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    ar[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Every wavefront walks its K range from a different starting chunk (and wraps
  // around): rows lie K floats apart, so waves that moved through K in step
  // would all hit the same few HBM channels at once.
  const int nch = (kend - kbeg + 16 * U - 1) / (16 * U);
  int ch = (int)((blockIdx.x * 4u + (threadIdx.x >> 6)) % (unsigned)nch);
  for (int it = 0; it < nch; ++it) {
    const int k0 = kbeg + ch * 16 * U;
    ch = (ch + 1 == nch) ? 0 : ch + 1;
    float4 w[U][NB], c[U], r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 16 * u + 4 * g;
      const bool kok = k < kend;  // K and kchunk are multiples of 4
      const long long kc = kok ? k : kbeg;
#pragma unroll
      for (int b = 0; b < NB; ++b) w[u][b] = ldg4(d.W, wrow[b] + kc);
      if (AMODE == A_IBP_BOX) {
        const float4 l = ldg4(d.A, xrow + kc), h = ldg4(d.A2, xrow + kc);
        c[u] = make_float4((l.x + h.x) * 0.5f, (l.y + h.y) * 0.5f, (l.z + h.z) * 0.5f, (l.w + h.w) * 0.5f);
        r[u] = make_float4((h.x - l.x) * 0.5f, (h.y - l.y) * 0.5f, (h.z - l.z) * 0.5f, (h.w - l.w) * 0.5f);
      } else {
        c[u] = ldg4(d.A, xrow + kc);
        r[u] = d.A2 ? ldg4(d.A2, xrow + kc) : make_float4(d.eps, d.eps, d.eps, d.eps);
      }
      if (!(kok && jok)) {
        c[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        r[u] = c[u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float cs[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
      const float rs[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float4& wv = w[u][b];
          const float ws = s == 0 ? wv.x : s == 1 ? wv.y : s == 2 ? wv.z : wv.w;
          ac[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(ws, cs[s], ac[b], 0, 0, 0);
          ar[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(fabsf(ws), rs[s], ar[b], 0, 0, 0);
        }
      }
    }
  }
  // result register v of lane (r16, g): neuron n0 + 16*blk + 4*g + v, input r16
  if (!jok) return;
  const long long MN = (long long)d.batch * d.N;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int n = n0 + 16 * b + 4 * g + v;
      if (n >= d.N) continue;
      const long long o = (long long)r16 * d.N + n;
      if (d.pc) {
        d.pc[blockIdx.y * MN + o] = ac[b][v];
        d.pr[blockIdx.y * MN + o] = ar[b][v];
      } else {
        const float cc = ac[b][v] + (d.bias ? d.bias[n] : 0.f);
        const float l = cc - ar[b][v], u = cc + ar[b][v];
        d.lo[o] = l;
        d.hi[o] = u;
        if (d.relu_lo) {
          d.relu_lo[o] = fmaxf(l, 0.f);
          d.relu_hi[o] = fmaxf(u, 0.f);
        }
      }
    }
  }
}

// Sum of the slice partials of one output (b, n) per wavefront, in a fixed
// order (lane-strided sums, then a shuffle tree), + bias, ReLU copies.
__global__ __launch_bounds__(256) void narrow_finish_kernel(const float* __restrict__ pc,
                                                            const float* __restrict__ pr, int S, long long MN,
                                                            int N, const float* __restrict__ bias,
                                                            float* __restrict__ lo, float* __restrict__ hi,
                                                            float* __restrict__ rlo, float* __restrict__ rhi) {
  const long long e = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= MN) return;
  const int lane = threadIdx.x & 63;
  float c = 0.f, r = 0.f;
  for (int q = lane; q < S; q += 64) {
    c += pc[q * MN + e];
    r += pr[q * MN + e];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    c += __shfl_xor(c, o, 64);
    r += __shfl_xor(r, o, 64);
  }
  if (lane != 0) return;
  c += bias ? bias[e % N] : 0.f;
  const float l = c - r, u = c + r;
  lo[e] = l;
  hi[e] = u;
  if (rlo) {
    rlo[e] = fmaxf(l, 0.f);
    rhi[e] = fmaxf(u, 0.f);
  }
}

}  // namespace

bool ibp_narrow_fits(int batch, int K, const float* W, const float* A, const float* A2) {
  auto al = [](const float* p) { return ((uintptr_t)p & 15) == 0; };
  return batch >= 1 && batch <= 16 && K >= 4 && K % 4 == 0 && al(W) && al(A) && (!A2 || al(A2));
}

int ibp_narrow_slices(int N, int K) {
  const long long waves = (N + ROWS - 1) / ROWS;
  int S = 1;
  // four wavefronts for every SIMD, slices of >= 256 K
  while (waves * S < 4096 && K / (2 * S) >= 256) S *= 2;
  return S;
}

hipError_t launch_ibp_narrow(NarrowIbp d, int S, hipStream_t st) {
  if (d.N <= 0 || d.batch <= 0) return hipSuccess;
  d.kchunk = ((d.K + S - 1) / S + 15) / 16 * 16;
  const int slices = (d.K + d.kchunk - 1) / d.kchunk;
  if (slices > 1 && !d.pc) return hipErrorInvalidValue;
  if (slices == 1) d.pc = d.pr = nullptr;
  const unsigned waves = (unsigned)((d.N + ROWS - 1) / ROWS);
  const dim3 grid((waves + 3) / 4, (unsigned)slices);
  if (d.amode == A_IBP_BOX)
    hipLaunchKernelGGL(ibp_narrow_kernel<A_IBP_BOX>, grid, dim3(256), 0, st, d);
  else
    hipLaunchKernelGGL(ibp_narrow_kernel<A_IBP_BALL>, grid, dim3(256), 0, st, d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || slices == 1) return e;
  const long long MN = (long long)d.batch * d.N;
  if (slices < 64)
    return launch_ibp_splitk_finish(d.pc, d.pr, slices, MN, d.N, d.bias, d.lo, d.hi, d.relu_lo, d.relu_hi, st);
  hipLaunchKernelGGL(narrow_finish_kernel, dim3((unsigned)((MN + 3) / 4)), dim3(256), 0, st, d.pc, d.pr, slices, MN,
                     d.N, d.bias, d.lo, d.hi, d.relu_lo, d.relu_hi);
  return hipGetLastError();
}

}  // namespace vb

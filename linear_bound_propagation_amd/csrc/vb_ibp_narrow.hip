// Interval bound propagation (centre/radius form) through one Linear layer for
// a small batch, the case where the weight matrix is read from HBM once and
// dominates all traffic (the page's wide single-hidden-layer networks, Sec. 1;
// IBP as the cheap bound of Sec. 2.1).
//
// Two options cut the kernel's work per weight byte.  (1) A packed copy of the
// weights (vb_pack_linear) stores each 16-row x 16-column block as 1 KB in the
// order the lanes read it, so every load instruction covers 1 KB of contiguous
// memory instead of 64-byte pieces of 16 rows.  (2) For a ball of one radius
// (the input layer), |W| r is eps times the row sums of |W|, the same for every
// input: they are added on the vector ALUs from the weight registers and the
// second MFMA chain is dropped.
// Output neurons run along the MFMA row dimension and the batch along its
// column dimension (v_mfma_f32_16x16x4f32, at most 16 inputs): each lane
// streams float4 pieces of its weight rows straight from HBM into registers
// (no LDS staging, nothing is reused), and the input centres / radii, which
// every wave reads, come from L2.  (A variant that read 128 x 64 weight tiles
// with every load instruction covering 256 contiguous bytes of four rows and
// went through LDS into the operand layout ran at 4.0 TB/s against 4.8 TB/s for
// this one: with its 70 KB of LDS per workgroup it kept half as many bytes in
// flight per CU.)  One chain of MFMAs accumulates W.c, a second
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
constexpr int U = 4;           // 16-wide K steps whose loads are issued together: a lane's
                               // four float4 of a row and its row's other three lanes cover
                               // 256 contiguous bytes of that row per step

// float4 at a clamped element offset (always a valid address of the array)
__device__ __forceinline__ float4 ldg4(const float* __restrict__ p, long long off) {
  return *reinterpret_cast<const float4*>(p + off);
}
// the same, non-temporal: packed weight blocks are read once per call and
// streamed past the caches (with row-major rows, whose lines are revisited by
// the next K steps, it was slower)
__device__ __forceinline__ float4 ldg4_nt(const float* __restrict__ p, long long off) {
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + off));
  return make_float4(t.x, t.y, t.z, t.w);
}

template <int AMODE, bool PACK, bool RS>
__global__ __launch_bounds__(256) void ibp_narrow_kernel(NarrowIbp d) {
  const int lane = threadIdx.x & 63;
  // wavefronts are numbered over (slice, block of ROWS neurons), so a layer with
  // few neurons and many slices still fills every workgroup
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nrb = (d.N + ROWS - 1) / ROWS;
  const int slice = wid / nrb;
  if (slice >= d.slices) return;  // whole wavefront; the kernel has no barriers
  const int n0 = (wid - slice * nrb) * ROWS;
  const int r16 = lane & 15, g = lane >> 4;
  const int kbeg = slice * d.kchunk;
  const int kend = min(d.K, kbeg + d.kchunk);
  // A operand: lane (r16, g) holds weight row n0 + 16*blk + r16 and K index
  // 4*g + s of every 16-wide step s; B operand: input r16 at the same K index.
  const bool jok = r16 < d.batch;
  const long long xrow = (long long)(jok ? r16 : 0) * d.K;
  // row-major: the element offset of each of this lane's rows; packed: of the
  // lane's float4 in the first 16-column block of each of its 16-row blocks
  // (the packed copy holds whole blocks, rows past N zero)
  long long wrow[NB];
  const int KT = d.K / 16, nblk = (d.N + 15) / 16;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (PACK) {
      const int rb = min((n0 >> 4) + b, nblk - 1);
      wrow[b] = (long long)rb * KT * 256 + lane * 4;
    } else {
      const int n = n0 + 16 * b + r16;
      wrow[b] = (long long)(n < d.N ? n : d.N - 1) * d.K;
    }
  }
  f32x4 ac[NB], ar[NB];
  float rs[NB];  // (RS) partial sums of |W| over this lane's columns of its rows
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    ac[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    ar[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    rs[b] = 0.f;
  }
  // Every wavefront walks its K range from a different starting chunk (and wraps
  // around): rows lie K floats apart, so waves that moved through K in step
  // would all hit the same few HBM channels at once.
  const int nch = (kend - kbeg + 16 * U - 1) / (16 * U);
  int ch = (int)((unsigned)wid % (unsigned)nch);
  for (int it = 0; it < nch; ++it) {
    const int k0 = kbeg + ch * 16 * U;
    ch = (ch + 1 == nch) ? 0 : ch + 1;
    float4 w[U][NB], c[U], r[U];
    bool kin[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 16 * u + 4 * g;
      const bool kok = k < kend;  // K and kchunk are multiples of 4 (of 16 with PACK: kok is per u)
      kin[u] = kok;
      const long long kc = kok ? k : kbeg;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // (a 16-row block wholly past N adds nothing that is stored: no load)
        if (n0 + 16 * b >= d.N) {
          w[u][b] = make_float4(0.f, 0.f, 0.f, 0.f);
          continue;
        }
        w[u][b] = PACK ? ldg4_nt(d.W, wrow[b] + (long long)((kok ? k0 + 16 * u : kbeg) >> 4) * 256)
                       : ldg4(d.W, wrow[b] + kc);
      }
      if (AMODE == A_IBP_BOX) {
        const float4 l = ldg4(d.A, xrow + kc), h = ldg4(d.A2, xrow + kc);
        c[u] = make_float4((l.x + h.x) * 0.5f, (l.y + h.y) * 0.5f, (l.z + h.z) * 0.5f, (l.w + h.w) * 0.5f);
        r[u] = make_float4((h.x - l.x) * 0.5f, (h.y - l.y) * 0.5f, (h.z - l.z) * 0.5f, (h.w - l.w) * 0.5f);
      } else {
        c[u] = ldg4(d.A, xrow + kc);
        r[u] = (!RS && d.A2) ? ldg4(d.A2, xrow + kc) : make_float4(d.eps, d.eps, d.eps, d.eps);
      }
      if (!(kok && jok)) {
        c[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        r[u] = c[u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float cs[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
      const float rs_[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float4& wv = w[u][b];
          const float ws = s == 0 ? wv.x : s == 1 ? wv.y : s == 2 ? wv.z : wv.w;
          ac[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(ws, cs[s], ac[b], 0, 0, 0);
          if (!RS) ar[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(fabsf(ws), rs_[s], ar[b], 0, 0, 0);
        }
      }
      if (RS && kin[u]) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          rs[b] += (fabsf(w[u][b].x) + fabsf(w[u][b].y)) + (fabsf(w[u][b].z) + fabsf(w[u][b].w));
      }
    }
  }
  if (RS) {
    // row sums of |W| of row 16 b + r16 over the four column groups, then the
    // sum of the row this lane's results belong to (neuron 16 b + 4 g + v: lane 4 g + v)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      rs[b] += __shfl_xor(rs[b], 16, 64);
      rs[b] += __shfl_xor(rs[b], 32, 64);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) ar[b][v] = d.eps * __shfl(rs[b], 4 * g + v, 64);
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
        // (many slices: partials of one output next to each other, for the finish)
        const long long po = d.slices >= 64 ? o * d.slices + slice : slice * MN + o;
        d.pc[po] = ac[b][v];
        d.pr[po] = ar[b][v];
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
// order (lane-strided sums, then a shuffle tree), + bias, ReLU copies.  The S
// partials of output e are contiguous at e * S.
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
    c += pc[e * S + q];
    r += pr[e * S + q];
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
  // two wavefronts for every SIMD (the kernel's register budget allows two:
  // a second round of workgroups would start in step with the first), slices
  // of >= 128 K (two load batches)
  while (waves * S < 2048 && K / (2 * S) >= 128) S *= 2;
  return S;
}

hipError_t launch_ibp_narrow(NarrowIbp d, int S, hipStream_t st) {
  if (d.N <= 0 || d.batch <= 0) return hipSuccess;
  d.kchunk = ((d.K + S - 1) / S + 15) / 16 * 16;
  const int slices = (d.K + d.kchunk - 1) / d.kchunk;
  if (slices > 1 && !d.pc) return hipErrorInvalidValue;
  if (slices == 1) d.pc = d.pr = nullptr;
  d.slices = slices;
  const long long waves = (long long)((d.N + ROWS - 1) / ROWS) * slices;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (d.packed && d.K % 16 != 0) return hipErrorInvalidValue;
  // radius by row sums: a ball of one radius only
  const bool rs = d.amode == A_IBP_BALL && d.A2 == nullptr;
  if (d.amode == A_IBP_BOX) {
    if (d.packed)
      hipLaunchKernelGGL((ibp_narrow_kernel<A_IBP_BOX, true, false>), grid, dim3(256), 0, st, d);
    else
      hipLaunchKernelGGL((ibp_narrow_kernel<A_IBP_BOX, false, false>), grid, dim3(256), 0, st, d);
  } else if (rs) {
    if (d.packed)
      hipLaunchKernelGGL((ibp_narrow_kernel<A_IBP_BALL, true, true>), grid, dim3(256), 0, st, d);
    else
      hipLaunchKernelGGL((ibp_narrow_kernel<A_IBP_BALL, false, true>), grid, dim3(256), 0, st, d);
  } else {
    if (d.packed)
      hipLaunchKernelGGL((ibp_narrow_kernel<A_IBP_BALL, true, false>), grid, dim3(256), 0, st, d);
    else
      hipLaunchKernelGGL((ibp_narrow_kernel<A_IBP_BALL, false, false>), grid, dim3(256), 0, st, d);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || slices == 1) return e;
  const long long MN = (long long)d.batch * d.N;
  if (slices < 64)
    return launch_ibp_splitk_finish(d.pc, d.pr, slices, MN, d.N, d.bias, d.lo, d.hi, d.relu_lo, d.relu_hi, st);
  hipLaunchKernelGGL(narrow_finish_kernel, dim3((unsigned)((MN + 3) / 4)), dim3(256), 0, st, d.pc, d.pr, slices, MN,
                     d.N, d.bias, d.lo, d.hi, d.relu_lo, d.relu_hi);
  return hipGetLastError();
}

// Packed copy of W [N][K] for the narrow kernel: block (rb, kc) of rows 16 rb
// .. 16 rb + 15 and columns 16 kc .. 16 kc + 15 at floats (rb K/16 + kc) 256,
// its float4 number l (lane l of the reading wavefront) holding row 16 rb +
// l % 16, columns 16 kc + 4 (l / 16) .. + 3; rows past N are zero.
__global__ void pack_linear_kernel(const float* __restrict__ W, int N, int K, float* __restrict__ dst) {
  const int KT = K / 16;
  const long long total = (long long)((N + 15) / 16) * 16 * K;
  for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (long long)gridDim.x * blockDim.x) {
    const long long blk = o >> 8;
    const int e = (int)(o & 255), l = e >> 2, comp = e & 3;
    const long long rb = blk / KT;
    const int kc = (int)(blk - rb * KT);
    const long long row = rb * 16 + (l & 15);
    dst[o] = row < N ? W[row * K + kc * 16 + 4 * (l >> 4) + comp] : 0.f;
  }
}

size_t pack_linear_floats(int N, int K) { return (size_t)((N + 15) / 16) * 16 * (size_t)K; }

hipError_t launch_pack_linear(const float* W, int N, int K, float* dst, hipStream_t st) {
  if (N <= 0 || K <= 0 || K % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_linear_kernel, dim3(8192), dim3(256), 0, st, W, N, K, dst);
  return hipGetLastError();
}

}  // namespace vb

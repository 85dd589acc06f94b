// Small HIP kernels of the bound propagation library (gfx950): row
// reductions, spec and identity row set-up, standalone relaxation and
// concretisation, IBP elementwise nodes, weight transposition, and the last
// back-substitution step onto a few-channel domain (on 16x16x4 matrix
// blocks).  The implicit GEMM lives in vb_gemm.hip.  All reductions run in a fixed order
// (wavefront shuffles, then a fixed combination of wavefronts), so results
// are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vb_internal.h"

namespace vb {

// ---------------------------------------------------------------------------
// reductions and elementwise kernels

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void relax_coeffs(float l, float u, float& a, float& s, float& t) {
  if (u <= 0.f) {
    a = 0.f; s = 0.f; t = 0.f;
  } else if (l >= 0.f) {
    a = 1.f; s = 1.f; t = 0.f;
  } else {
    s = u / (u - l);
    t = -s * l;
    a = (u >= -l) ? 1.f : 0.f;
  }
}

// Fixed-order block sum of one value per thread (256 threads); result valid in thread 0.
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x == 0) s = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(256) void rows_reduce_kernel(const float* __restrict__ part, int Z, int rows,
                                                          int P, int S, int ld, float* __restrict__ rowacc,
                                                          int accumulate, int pos_major) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int PS = P * S;
  const int L = Z * PS;
  float s = 0.f;
  for (int e = lane; e < L; e += 64) {
    int z = e / PS;
    int q = e - z * PS;
    int p = q / S;
    int c = q - p * S;
    s += pos_major ? part[(((long long)z * P + p) * rows + row) * ld + c]
                   : part[(((long long)z * rows + row) * P + p) * ld + c];
  }
  s = wave_sum(s);
  if (lane == 0) rowacc[row] = accumulate ? rowacc[row] + s : s;
}

// The same with one thread per row, for rows of few partials (a wavefront per
// row would leave most of its lanes idle): in the position-major layout the
// threads of a wavefront read consecutive rows of one (z, p, c).
__global__ __launch_bounds__(256) void rows_reduce_thread_kernel(const float* __restrict__ part, int Z, int rows,
                                                                 int P, int S, int ld, float* __restrict__ rowacc,
                                                                 int accumulate, int pos_major) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  float s = 0.f;
  for (int z = 0; z < Z; ++z)
    for (int p = 0; p < P; ++p)
      for (int c = 0; c < S; ++c)
        s += pos_major ? part[(((long long)z * P + p) * rows + row) * ld + c]
                       : part[(((long long)z * rows + row) * P + p) * ld + c];
  rowacc[row] = accumulate ? rowacc[row] + s : s;
}

hipError_t launch_rows_reduce(const float* part, int Z, int rows, int P, int S, int ld, float* rowacc,
                              int accumulate, int pos_major, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if ((long long)Z * P * S <= 64)
    hipLaunchKernelGGL(rows_reduce_thread_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, part, Z, rows, P, S,
                       ld, rowacc, accumulate, pos_major);
  else
    hipLaunchKernelGGL(rows_reduce_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, part, Z, rows, P, S, ld,
                       rowacc, accumulate, pos_major);
  return hipGetLastError();
}

__global__ void finish_kernel(const float* __restrict__ acc, int batch, int R, float* lb, float* ub,
                              float* best, int intersect) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)batch * R) return;
  const long long b = i / R, r = i - b * R;
  const float l = acc[b * 2 * R + r];
  const float u = -acc[b * 2 * R + R + r];
  if (lb) lb[i] = intersect ? fmaxf(lb[i], l) : l;
  if (ub) ub[i] = intersect ? fminf(ub[i], u) : u;
  if (best) best[i] = fmaxf(best[i], l);
}

hipError_t launch_finish(const float* rowacc, int batch, int R, float* lb, float* ub, float* best,
                         hipStream_t st, int intersect) {
  long long n = (long long)batch * R;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(finish_kernel, dim3((n + 255) / 256), dim3(256), 0, st, rowacc, batch, R, lb, ub, best,
                     intersect);
  return hipGetLastError();
}

__global__ void finish_lower_kernel(const float* __restrict__ acc, long long n, float* lb, float* best, int init) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float l = acc[i];
  if (lb) lb[i] = l;
  if (best) best[i] = init ? l : fmaxf(best[i], l);
}

hipError_t launch_finish_lower(const float* rowacc, long long n, float* lb, float* best, int init, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(finish_lower_kernel, dim3((n + 255) / 256), dim3(256), 0, st, rowacc, n, lb, best, init);
  return hipGetLastError();
}

// one wave per spec row
__global__ __launch_bounds__(256) void spec_init_kernel(const float* __restrict__ C, int batch, int m, int n,
                                                        const float* __restrict__ bias, int bias_c,
                                                        float* __restrict__ lam, float* __restrict__ rowacc,
                                                        int split) {
  const int RR = split ? 2 * m : m;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (long long)batch * RR) return;
  const long long b = row / RR;
  const int r = (int)(row - b * RR);
  const float sg = (r < m) ? 1.f : -1.f;
  const float* src = C + (b * m + (r < m ? r : r - m)) * (long long)n;
  float* dst = lam + row * n;
  float s = 0.f;
  for (int j = lane; j < n; j += 64) {
    float v = sg * src[j];
    dst[j] = v;
    if (bias) s += v * bias[j % bias_c];
  }
  s = wave_sum(s);
  if (lane == 0) rowacc[row] = s;
}

hipError_t launch_spec_init(const float* C, int batch, int m, int n, const float* bias, int bias_c, float* lam,
                            float* rowacc, int split, hipStream_t st) {
  long long rows = (long long)batch * (split ? 2 * m : m);
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(spec_init_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, C, batch, m, n, bias,
                     bias_c > 0 ? bias_c : n, lam, rowacc, split);
  return hipGetLastError();
}

// one wave per identity row (b, sign, i)
__global__ __launch_bounds__(256) void identity_linear_kernel(const float* __restrict__ W, int n_out, int n_in,
                                                              const float* __restrict__ bias_start,
                                                              const float* __restrict__ lo,
                                                              const float* __restrict__ hi,
                                                              const float* __restrict__ bias_z, int bias_zc,
                                                              int batch, float* __restrict__ lam,
                                                              float* __restrict__ rowacc, const int* __restrict__ sel,
                                                              const int* __restrict__ cnt, int U) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nr = sel ? U : n_out;  // rows per sign
  const int R = 2 * nr;
  if (row >= (long long)batch * R) return;
  const long long b = row / R;
  const int r = (int)(row - b * R);
  const int u = r < nr ? r : r - nr;
  const float sg = r < nr ? 1.f : -1.f;
  float* dst = lam + row * n_in;
  if (sel && u >= cnt[b]) {
    // past this input's count of selected neurons: a zero row
    for (int j = lane; j < n_in; j += 64) dst[j] = 0.f;
    if (lane == 0) rowacc[row] = 0.f;
    return;
  }
  const int i = sel ? sel[b * n_out + u] : u;
  const float* w = W + (long long)i * n_in;
  const float* lb = lo + b * n_in;
  const float* ub = hi + b * n_in;
  float s = 0.f;
  for (int j = lane; j < n_in; j += 64) {
    float psi = sg * w[j];
    float a, sl, t;
    relax_coeffs(lb[j], ub[j], a, sl, t);
    float o = psi >= 0.f ? psi * a : psi * sl;
    dst[j] = o;
    if (bias_z) s += o * bias_z[j % bias_zc];
    s += fminf(psi, 0.f) * t;
  }
  s = wave_sum(s);
  if (lane == 0) rowacc[row] = (bias_start ? sg * bias_start[i] : 0.f) + s;
}

// The same rows, a workgroup per (input b, IL_RI neurons) (with a neuron list,
// rows past the input's count are not written): the relaxation
// coefficients of b's neurons are worked out once per column and serve the
// 2 * IL_RI rows (both signs) of the group, each weight float4 is loaded once
// for its two rows, and every access is a 16-byte one (n_in % 4 == 0).  A
// row's sum runs over its columns in the same order whichever rows share the
// workgroup (thread-strided float4 columns, then a fixed-order block sum).
constexpr int IL_RI = 8;

__global__ __launch_bounds__(256) void identity_linear4_kernel(const float* __restrict__ W, int n_out, int n_in,
                                                               const float* __restrict__ bias_start,
                                                               const float* __restrict__ lo,
                                                               const float* __restrict__ hi,
                                                               const float* __restrict__ bias_z, int bias_zc,
                                                               float* __restrict__ lam, float* __restrict__ rowacc,
                                                               const int* __restrict__ sel,
                                                               const int* __restrict__ cnt, int U) {
  const int nr = sel ? U : n_out;  // rows per sign
  const int groups = (nr + IL_RI - 1) / IL_RI;
  const int b = blockIdx.x / groups;
  const int u0 = (blockIdx.x - b * groups) * IL_RI;
  const int tid = threadIdx.x;
  const int nb = sel ? cnt[b] : nr;  // live rows of this input
  // rows past the live count are never read (their GEMM tiles return at once,
  // the finishing step skips them): a group with no live row writes nothing
  if (u0 >= nb) return;
  int src[IL_RI];
#pragma unroll
  for (int q = 0; q < IL_RI; ++q) {
    const int u = u0 + q;
    src[q] = u < nb ? (sel ? sel[(long long)b * n_out + u] : u) : -1;
  }
  const long long rp = (long long)b * 2 * nr + u0, rm = rp + nr;  // first + and - row
  float sp[IL_RI], sm[IL_RI];
#pragma unroll
  for (int q = 0; q < IL_RI; ++q) sp[q] = sm[q] = 0.f;
  const float* lb = lo + (long long)b * n_in;
  const float* ub = hi + (long long)b * n_in;
  for (int j = 4 * tid; j < n_in; j += 1024) {
    const float4 l4 = *reinterpret_cast<const float4*>(lb + j);
    const float4 h4 = *reinterpret_cast<const float4*>(ub + j);
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, hv[4] = {h4.x, h4.y, h4.z, h4.w};
    float a[4], sl[4], t[4], bz[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      relax_coeffs(lv[e], hv[e], a[e], sl[e], t[e]);
      bz[e] = bias_z ? bias_z[(j + e) % bias_zc] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < IL_RI; ++q) {
      if (u0 + q >= nb) break;
      const float4 w4 = *reinterpret_cast<const float4*>(W + (long long)src[q] * n_in + j);
      const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
      float op[4], om[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pp = wv[e], pm = -wv[e];
        op[e] = pp >= 0.f ? pp * a[e] : pp * sl[e];
        om[e] = pm >= 0.f ? pm * a[e] : pm * sl[e];
        if (bias_z) {
          sp[q] += op[e] * bz[e];
          sm[q] += om[e] * bz[e];
        }
        sp[q] += fminf(pp, 0.f) * t[e];
        sm[q] += fminf(pm, 0.f) * t[e];
      }
      *reinterpret_cast<float4*>(lam + (rp + q) * n_in + j) = make_float4(op[0], op[1], op[2], op[3]);
      *reinterpret_cast<float4*>(lam + (rm + q) * n_in + j) = make_float4(om[0], om[1], om[2], om[3]);
    }
  }
  __shared__ float red[4][2 * IL_RI];
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int q = 0; q < IL_RI; ++q) {
    const float x = wave_sum(sp[q]), y = wave_sum(sm[q]);
    if (lane == 0) {
      red[wv][q] = x;
      red[wv][IL_RI + q] = y;
    }
  }
  __syncthreads();
  if (tid < 2 * IL_RI) {
    const int q = tid % IL_RI;
    const bool minus = tid >= IL_RI;
    if (u0 + q < nb) {
      const float tot = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
      const float sg = minus ? -1.f : 1.f;
      rowacc[(minus ? rm : rp) + q] = (bias_start ? sg * bias_start[src[q]] : 0.f) + tot;
    }
  }
}

hipError_t launch_identity_linear(const float* W, int n_out, int n_in, const float* bias_start, const float* lo,
                                  const float* hi, const float* bias_z, int bias_zc, int batch, float* lam,
                                  float* rowacc, hipStream_t st, const int* sel, const int* cnt, int U) {
  long long rows = (long long)batch * 2 * (sel ? U : n_out);
  if (rows <= 0) return hipSuccess;
  auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (n_in % 4 == 0 && al(W) && al(lo) && al(hi) && al(lam)) {
    const long long groups = ((sel ? U : n_out) + IL_RI - 1) / IL_RI;
    hipLaunchKernelGGL(identity_linear4_kernel, dim3((unsigned)(batch * groups)), dim3(256), 0, st, W, n_out, n_in,
                       bias_start, lo, hi, bias_z, bias_zc > 0 ? bias_zc : n_in, lam, rowacc, sel, cnt, U);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(identity_linear_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, W, n_out, n_in,
                     bias_start, lo, hi, bias_z, bias_zc > 0 ? bias_zc : n_in, batch, lam, rowacc, sel, cnt, U);
  return hipGetLastError();
}

// Selected identity rows written out: row (b, sign, u) is sign * e_{sel[b][u]} over n
// neurons (zero when u >= cnt[b]); rowacc = sign * bias[sel] (0 when padding).
__global__ __launch_bounds__(256) void select_fill_kernel(int batch, int n, int U, const int* __restrict__ sel,
                                                          const int* __restrict__ cnt, const float* __restrict__ bias,
                                                          int bias_c, float* __restrict__ lam,
                                                          float* __restrict__ rowacc) {
  const long long rows = (long long)batch * 2 * U;
  for (long long row = blockIdx.x; row < rows; row += gridDim.x) {
    const long long b = row / (2 * U);
    const int r = (int)(row - b * 2 * U);
    const int u = r < U ? r : r - U;
    const float sg = r < U ? 1.f : -1.f;
    const int col = u < cnt[b] ? sel[b * n + u] : -1;
    float* out = lam + row * n;
    for (int e = threadIdx.x; e < n; e += 256) out[e] = e == col ? sg : 0.f;
    if (threadIdx.x == 0) rowacc[row] = (col >= 0 && bias) ? sg * bias[col % bias_c] : 0.f;
  }
}

hipError_t launch_select_fill(int batch, int n, int U, const int* sel, const int* cnt, const float* bias, int bias_c,
                              float* lam, float* rowacc, hipStream_t st) {
  const long long rows = (long long)batch * 2 * U;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(select_fill_kernel, dim3((unsigned)std::min<long long>(rows, 65536)), dim3(256), 0, st, batch, n,
                     U, sel, cnt, bias, bias_c > 0 ? bias_c : n, lam, rowacc);
  return hipGetLastError();
}

// sel[b][rank] = j for every neuron j with idx[b][j] = rank >= 0 (the inverse of a ranking)
__global__ void rank_to_list_kernel(const int* __restrict__ idx, long long total, int n, int* __restrict__ sel) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long long)gridDim.x * blockDim.x) {
    const int r = idx[e];
    if (r >= 0) sel[(e / n) * n + r] = (int)(e % n);
  }
}

hipError_t launch_rank_to_list(const int* idx, int batch, int n, int* sel, hipStream_t st) {
  const long long total = (long long)batch * n;
  if (total <= 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(rank_to_list_kernel, dim3((unsigned)blocks), dim3(256), 0, st, idx, total, n, sel);
  return hipGetLastError();
}

// Bounds of the selected neurons from their rows (2U per input: +e then -e):
// lb[b][sel] = acc (or the max with the value there), ub[b][sel] = -acc (or the min).
__global__ void finish_select_kernel(const float* __restrict__ acc, int batch, int U, int n,
                                     const int* __restrict__ sel, const int* __restrict__ cnt, float* lb, float* ub,
                                     int intersect) {
  const long long total = (long long)batch * U;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long long)gridDim.x * blockDim.x) {
    const long long b = e / U;
    const int u = (int)(e - b * U);
    if (u >= cnt[b]) continue;
    const long long j = b * n + sel[b * n + u];
    const float l = acc[b * 2 * U + u], h = -acc[b * 2 * U + U + u];
    if (lb) lb[j] = intersect ? fmaxf(lb[j], l) : l;
    if (ub) ub[j] = intersect ? fminf(ub[j], h) : h;
  }
}

hipError_t launch_finish_select(const float* acc, int batch, int U, int n, const int* sel, const int* cnt, float* lb,
                                float* ub, int intersect, hipStream_t st) {
  const long long total = (long long)batch * U;
  if (total <= 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(finish_select_kernel, dim3((unsigned)blocks), dim3(256), 0, st, acc, batch, U, n, sel, cnt, lb,
                     ub, intersect);
  return hipGetLastError();
}

// one block per identity row; the element index runs in 32 bits and advances
// by the block size without a division per element (but one by Wi)
__global__ __launch_bounds__(256) void identity_conv_kernel(const IdConv a, float* __restrict__ rowacc) {
  __shared__ float sh[4];
  const long long row = blockIdx.x;
  const long long n_out = (long long)a.Co * a.Ho * a.Wo;
  const long long R = 2 * n_out;
  const long long b = row / R;
  const long long r = row - b * R;
  const float sg = r < n_out ? 1.f : -1.f;
  const long long i = r < n_out ? r : r - n_out;
  const int c = (int)(i % a.Co);
  const int p = (int)(i / a.Co);
  const int y = p / a.Wo, x = p - (p / a.Wo) * a.Wo;
  const int L = a.Hi * a.Wi * a.Ci;
  const float* addend = a.addend ? a.addend + row * L : nullptr;
  float* out = a.out ? a.out + row * L : nullptr;
  const float* lo = a.lo ? a.lo + b * L : nullptr;
  const float* hi = a.hi ? a.hi + b * L : nullptr;
  const float* center = a.center ? a.center + b * L : nullptr;
  const float* radius = a.radius ? a.radius + b * L : nullptr;
  const int dq = 256 / a.Ci, dci = 256 - dq * a.Ci;
  int ci = threadIdx.x % a.Ci, q = threadIdx.x / a.Ci;
  float s = 0.f;
  for (int e = threadIdx.x; e < L; e += 256) {
    const int yy = q / a.Wi, xx = q - (q / a.Wi) * a.Wi;
    const int ky = yy - y * a.stride + a.pad, kx = xx - x * a.stride + a.pad;
    float v = 0.f;
    if (ky >= 0 && ky < a.kh && kx >= 0 && kx < a.kw) v = sg * a.W[((ky * a.kw + kx) * a.Co + c) * a.Ci + ci];
    if (addend) v += addend[e];
    if (a.mode == E_STORE) {
      out[e] = v;
      if (a.bias) s += v * a.bias[ci];
    } else if (a.mode == E_RELAX) {
      float al, sl, t;
      relax_coeffs(lo[e], hi[e], al, sl, t);
      const float o = v >= 0.f ? v * al : v * sl;
      out[e] = o;
      if (a.bias) s += o * a.bias[ci];
      s += fminf(v, 0.f) * t;
    } else {
      float cc, rr;
      if (center) {
        cc = center[e];
        rr = radius ? radius[e] : a.eps;
      } else {
        cc = (lo[e] + hi[e]) * 0.5f;
        rr = (hi[e] - lo[e]) * 0.5f;
      }
      s += v * cc - fabsf(v) * rr;
    }
    // next element: e + 256 = (q + dq) * Ci + (ci + dci), with a carry
    ci += dci;
    q += dq;
    if (ci >= a.Ci) {
      ci -= a.Ci;
      ++q;
    }
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) rowacc[row] += s;
}

hipError_t launch_identity_conv(const IdConv& a, int batch, float* rowacc, hipStream_t st) {
  const long long rows = (long long)batch * 2 * a.Co * a.Ho * a.Wo;
  if (rows <= 0) return hipSuccess;
  if ((long long)a.Hi * a.Wi * a.Ci >= (1LL << 31) - 256 || rows > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(identity_conv_kernel, dim3((unsigned)rows), dim3(256), 0, st, a, rowacc);
  return hipGetLastError();
}

// one block per row
__global__ __launch_bounds__(256) void col2im_kernel(const Col2Im a, float* __restrict__ rowacc) {
  __shared__ float sh[4];
  const long long row = blockIdx.x;
  const long long b = row / a.rows_per_b;
  const long long L = (long long)a.Hi * a.Wi * a.Ci;
  const int NQ = a.kh * a.kw * a.Ci;
  const float* q = a.Q + row * (long long)a.Ho * a.Wo * NQ;
  float s = 0.f;
  for (long long e = threadIdx.x; e < L; e += 256) {
    const int ci = (int)(e % a.Ci);
    const long long p = e / a.Ci;
    const int y = (int)(p / a.Wi), x = (int)(p % a.Wi);
    float v = 0.f;
    for (int ky = 0; ky < a.kh; ++ky) {
      const int ty = y + a.pad - ky;
      if (ty < 0 || ty % a.stride) continue;
      const int oy = ty / a.stride;
      if (oy >= a.Ho) continue;
      for (int kx = 0; kx < a.kw; ++kx) {
        const int tx = x + a.pad - kx;
        if (tx < 0 || tx % a.stride) continue;
        const int ox = tx / a.stride;
        if (ox >= a.Wo) continue;
        v += q[((long long)oy * a.Wo + ox) * NQ + (ky * a.kw + kx) * a.Ci + ci];
      }
    }
    if (a.addend) v += a.addend[row * L + e];
    if (a.psi_out) a.psi_out[row * L + e] = v;
    if (a.mode == E_STORE) {
      a.out[row * L + e] = v;
      if (a.bias) s += v * a.bias[ci];
    } else if (a.mode == E_RELAX) {
      const float l = a.lo[b * L + e], u = a.hi[b * L + e];
      float al, sl, t;
      relax_coeffs(l, u, al, sl, t);
      const float o = v >= 0.f ? v * al : v * sl;
      a.out[row * L + e] = o;
      if (a.bias) s += o * a.bias[ci];
      s += fminf(v, 0.f) * t;
    } else if (a.patch) {
      // window cell -> pixel of the domain node for this row's position
      const long long pz = (row / a.pc) % ((long long)a.pgh * a.pgw);
      const int py = (int)(pz / a.pgw), px = (int)(pz % a.pgw);
      const int ay = py * a.psy + a.poy + y, ax = px * a.psx + a.pox + x;
      if (ay >= 0 && ay < a.img_h && ax >= 0 && ax < a.img_w) {
        const long long ei = (b * a.img_h * a.img_w + (long long)ay * a.img_w + ax) * a.Ci + ci;
        const float c = a.center[ei];
        const float r = a.radius ? a.radius[ei] : a.eps;
        s += v * c - fabsf(v) * r;
      }
    } else {
      const float c = a.center[b * L + e];
      const float r = a.radius ? a.radius[b * L + e] : a.eps;
      s += v * c - fabsf(v) * r;
    }
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) rowacc[row] += s;
}

hipError_t launch_col2im(const Col2Im& a, int rows, float* rowacc, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(col2im_kernel, dim3(rows), dim3(256), 0, st, a, rowacc);
  return hipGetLastError();
}

namespace {
constexpr int CIN_THREADS = 256;         // threads of a conv-input workgroup, one input pixel each
constexpr int CIN_MAX_CO = 64;           // output channels: one 16-step pass of the contraction
constexpr int CIN_MB = 3;                // M-blocks whose loads are issued together
constexpr int CIN_WIN_ROWS = 16;         // footprint rows per workgroup
constexpr size_t CIN_Y_LDS = 64 * 1024;  // bytes of a band's tap table
typedef float cin_v4 __attribute__((ext_vector_type(4)));

// Columns of the tap table (tap x domain channel) in blocks of 16.
int cin_col_blocks(const ConvIn& a) { return (a.kh * a.kw * a.Ci + 15) / 16; }
// Floats per tap-table row: the columns, rounded up to an odd count so that
// threads reading consecutive rows hit distinct LDS banks.
__host__ __device__ inline int cin_row_floats(int ncol) { return ncol | 1; }

// Input rows per band: one output pixel per thread, and the tap table of the
// band's staged output rows within CIN_Y_LDS.
int cin_band_rows(const ConvIn& a) {
  const int ys = cin_row_floats(a.kh * a.kw * a.Ci);
  int bh = CIN_THREADS / a.Wi;
  if (bh > a.Hi) bh = a.Hi;
  while (bh >= 1) {
    const int nr = (bh + a.kh - 1 + a.stride - 1) / a.stride + 1;
    if ((size_t)nr * a.Wo * ys * sizeof(float) <= CIN_Y_LDS) return bh;
    --bh;
  }
  return 0;
}
}  // namespace

bool conv_input_fits(const ConvIn& a) {
  return a.Ci >= 1 && a.Ci <= 4 && a.Co % 16 == 0 && a.Co <= CIN_MAX_CO && a.Wi <= CIN_THREADS && a.stride >= 1 &&
         ((uintptr_t)a.W & 15) == 0 && ((uintptr_t)a.lam & 15) == 0 && cin_col_blocks(a) <= 3 &&
         cin_band_rows(a) >= 1;
}

size_t conv_input_part_floats(const ConvIn& a, int rows) {
  const int bh = cin_band_rows(a);
  return bh < 1 ? 0 : (size_t)rows * ((a.Hi + bh - 1) / bh);
}

// The last back-substitution step onto a few-channel domain on the matrix
// cores, in two phases per (row, band of input rows):
//  1. tap table Y[q][t * CI + ci] = sum_co Lambda[q][co] * W[t][co][ci] for
//     every staged output pixel q: a K = Co contraction with the (tap, domain
//     channel) pairs as N, on 16x16x4 fp32 blocks (A: pixel = lane % 16,
//     channel step = lane / 16; B: channel step = lane / 16, column = lane % 16;
//     result element (4 * (lane / 16) + v, lane % 16) in component v). Each
//     Lambda element is loaded once, straight from global memory.
//  2. each thread sums the taps that reach its input pixel from the table in
//     LDS, adds the addend, stores Psi if asked, and concretises.
// Consecutive workgroups go round-robin over the 8 XCDs; with xcd_map the
// bands of one row share an XCD, so the rows two bands both stage are read
// through one L2.
template <int CI, int NB, bool S1>
__global__ __launch_bounds__(CIN_THREADS) void conv_input_concretize_kernel(const ConvIn a, int BH, int nbands,
                                                                           int xcd_map, long long items,
                                                                           float* __restrict__ part) {
  extern __shared__ float ys[];  // [staged pixels][ysw]
  __shared__ float sh[CIN_THREADS / 64];
  constexpr int WAVES = CIN_THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntap = a.kh * a.kw;
  const int ncol = ntap * CI;
  const int ysw = cin_row_floats(ncol);
  const int li = lane & 15, kk = lane >> 4;

  // B of phase 1 (the same for every row): step j = 4u + c takes channel
  // 16u + 4 * (lane / 16) + c, so that one load instruction of A (fixed u)
  // reads 64 contiguous bytes of each of 16 pixels.
  float bw[NB][16];  // weights of column li of each block, 16 steps
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = nb * 16 + li;
    const bool okn = col < ncol;
    const int t = okn ? col / CI : 0, ci = okn ? col - t * CI : 0;
    const float* w = a.W + ((long long)t * a.Co + 4 * kk) * CI + ci;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int off = 16 * (j >> 2) + (j & 3);
      bw[nb][j] = okn && 16 * (j >> 2) < a.Co ? w[off * CI] : 0.f;
    }
  }

  // work item (row, band) n = blockIdx.x; with xcd_map the bands of one row
  // share an XCD
  {
  const long long n = (long long)blockIdx.x;
  if (n >= items) return;
  long long row;
  int band;
  if (xcd_map) {
    const unsigned slot = (unsigned)n >> 3, rb = slot / (unsigned)nbands;
    band = (int)(slot - rb * (unsigned)nbands);
    row = (long long)rb * 8 + (n & 7);
  } else {
    row = n / nbands;
    band = (int)(n - row * nbands);
  }
  const int y0 = band * BH, y1 = min(a.Hi, y0 + BH);
  const int s = S1 ? 1 : a.stride;
  const int lo = y0 + a.pad - (a.kh - 1);
  const int oy_lo = lo <= 0 ? 0 : (lo + s - 1) / s;
  const int oy_hi = min(a.Ho - 1, (y1 - 1 + a.pad) / s);
  const int nr = oy_hi - oy_lo + 1;
  const int npx = nr > 0 ? nr * a.Wo : 0;
  const float* lam_r = a.lam + (row * a.Ho + (nr > 0 ? oy_lo : 0)) * (long long)a.Wo * a.Co;

  // phase 1: tap table
  const int nmb = (npx + 15) / 16;
  const int nit = wave < nmb ? (nmb - wave + WAVES - 1) / WAVES : 0;  // M-blocks of this wavefront
  auto load_a = [&](int it, float4 (&v)[4]) {
    const int mb = wave + WAVES * it;
    // rows past the staged pixels are clamped (their results are never
    // stored); channel groups past Co are clamped and meet zero weights.
    // No load is predicated, so the waits before each M-block's products
    // cover only that block's loads.
    const int q = min(mb * 16 + li, npx - 1);
    const float4* ap = reinterpret_cast<const float4*>(lam_r + (long long)q * a.Co + 4 * kk);
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ap[16 * u < a.Co ? 4 * u : 0];
  };
  cin_v4 acc[NB];
  // the loads of up to CIN_MB M-blocks are issued together
  for (int g0 = 0; g0 < nit; g0 += CIN_MB) {
    float4 av[CIN_MB][4];
#pragma unroll
    for (int i = 0; i < CIN_MB; ++i) load_a(min(g0 + i, nit - 1), av[i]);
#pragma unroll
    for (int i = 0; i < CIN_MB; ++i) {
      if (g0 + i >= nit) break;
      const int mb = wave + WAVES * (g0 + i);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = cin_v4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float4 c4 = av[i][j >> 2];
        const float a1 = (j & 3) == 0 ? c4.x : (j & 3) == 1 ? c4.y : (j & 3) == 2 ? c4.z : c4.w;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bw[nb][j], acc[nb], 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int q = mb * 16 + 4 * kk + v;
        if (q < npx) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            if (nb * 16 + li < ncol) ys[q * ysw + nb * 16 + li] = acc[nb][v];
        }
      }
    }
  }
  __syncthreads();

  // phase 2: taps onto this thread's input pixel, concretisation
  float sum = 0.f;
  if (tid < (y1 - y0) * a.Wi) {
    const int py = y0 + tid / a.Wi, px = tid % a.Wi;
    float o[CI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) o[ci] = 0.f;
    for (int t = 0; t < ntap; ++t) {
      const int ky = t / a.kw, kx = t - ky * a.kw;
      const int ty = py + a.pad - ky, tx = px + a.pad - kx;
      int q = -1;
      if (ty >= 0 && tx >= 0) {
        if (S1) {
          if (ty <= oy_hi && tx < a.Wo) q = (ty - oy_lo) * a.Wo + tx;
        } else if (ty % s == 0 && tx % s == 0 && ty / s <= oy_hi && tx / s < a.Wo) {
          q = (ty / s - oy_lo) * a.Wo + tx / s;
        }
      }
      if (q >= 0) {
#pragma unroll
        for (int ci = 0; ci < CI; ++ci) o[ci] += ys[q * ysw + t * CI + ci];
      }
    }
    const long long b = row / a.rows_per_b;
    const long long pix = (long long)py * a.Wi + px;
    // the domain pixel of this input cell: itself, or for a footprint window
    // the cell's pixel at the row's position (none outside the image)
    long long dpix = b * a.Hi * a.Wi + pix;
    bool inside = true;
    if (a.patch) {
      const long long pz = (row / a.pc) % ((long long)a.pgh * a.pgw);
      const int gy = (int)(pz / a.pgw), gx = (int)(pz - (pz / a.pgw) * a.pgw);
      const int ay = gy * a.psy + a.poy + py, ax = gx * a.psx + a.pox + px;
      inside = ay >= 0 && ay < a.img_h && ax >= 0 && ax < a.img_w;
      dpix = b * a.img_h * a.img_w + (inside ? (long long)ay * a.img_w + ax : 0);
    }
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const long long e = (row * a.Hi * a.Wi + pix) * CI + ci;
      float v = o[ci];
      if (a.addend) v += a.addend[e];
      if (a.psi_out) a.psi_out[e] = v;
      const long long be = dpix * CI + ci;
      const float r = a.radius ? a.radius[be] : a.eps;
      if (inside) sum += v * a.center[be] - fabsf(v) * r;
    }
  }
  sum = wave_sum(sum);
  if (lane == 0) sh[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += sh[w];
    part[row * nbands + band] = t;
  }
  }
}

// Footprint windows (a window of at most 128 output cells per row, the whole
// window one band): the same two phases for P rows at once, so that small
// windows still occupy the workgroup.  Phase 1 spreads the P * ceil(cells/16)
// M-blocks (at most 8) over the four wavefronts, each tap table in its own LDS
// slice; in phase 2 thread t takes input pixel t % pix of row t / pix; each
// row's sum over its pixels is one wavefront's reduction.  The next group's
// Lambda is loaded while the current one computes; the weights stay in
// registers for all per_wg rows of the workgroup.
template <int CI, int NB, bool S1>
__global__ __launch_bounds__(CIN_THREADS) void conv_input_windows_kernel(const ConvIn a, int per_wg, int P,
                                                                        long long rows, float* __restrict__ part) {
  extern __shared__ float ys[];  // [P][cells][ysw]
  __shared__ float contrib[CIN_THREADS];
  constexpr int WAVES = CIN_THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntap = a.kh * a.kw;
  const int ncol = ntap * CI;
  const int ysw = cin_row_floats(ncol);
  const int li = lane & 15, kk = lane >> 4;
  const int cells = a.Ho * a.Wo, mbi = (cells + 15) / 16, pix = a.Hi * a.Wi;
  const int s = S1 ? 1 : a.stride;
  const int oy_hi = min(a.Ho - 1, (a.Hi - 1 + a.pad) / s);

  float bw[NB][16];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = nb * 16 + li;
    const bool okn = col < ncol;
    const int t = okn ? col / CI : 0, ci = okn ? col - t * CI : 0;
    const float* w = a.W + ((long long)t * a.Co + 4 * kk) * CI + ci;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int off = 16 * (j >> 2) + (j & 3);
      bw[nb][j] = okn && 16 * (j >> 2) < a.Co ? w[off * CI] : 0.f;
    }
  }

  const long long r_beg = (long long)blockIdx.x * per_wg;
  const long long r_end = min(rows, r_beg + per_wg);
  // M-block slot i of this wavefront in a group starting at row r0: item, block
  auto load_group = [&](long long r0, float4 (&v)[2][4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int gb = wave + WAVES * i;
      const int item = gb / mbi, mb = gb - item * mbi;
      long long row = r0 + item;
      if (row >= r_end) row = r_end - 1;  // clamped (never stored)
      const int q = min(mb * 16 + li, cells - 1);
      const float4* ap = reinterpret_cast<const float4*>(a.lam + (row * cells + q) * (long long)a.Co + 4 * kk);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[i][u] = ap[16 * u < a.Co ? 4 * u : 0];
    }
  };
  float4 nxa[2][4];
  if (r_beg < r_end) load_group(r_beg, nxa);
  for (long long r0 = r_beg; r0 < r_end; r0 += P) {
    float4 av[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) av[i][u] = nxa[i][u];
    if (r0 + P < r_end) load_group(r0 + P, nxa);
    // phase 1: tap tables of the group's rows
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int gb = wave + WAVES * i;
      const int item = gb / mbi, mb = gb - item * mbi;
      if (item >= P || r0 + item >= r_end) continue;
      cin_v4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = cin_v4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float4 c4 = av[i][j >> 2];
        const float a1 = (j & 3) == 0 ? c4.x : (j & 3) == 1 ? c4.y : (j & 3) == 2 ? c4.z : c4.w;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bw[nb][j], acc[nb], 0, 0, 0);
      }
      float* yt = ys + (long long)item * cells * ysw;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int q = mb * 16 + 4 * kk + v;
        if (q < cells) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            if (nb * 16 + li < ncol) yt[q * ysw + nb * 16 + li] = acc[nb][v];
        }
      }
    }
    __syncthreads();
    // phase 2: thread t -> input pixel t % pix of row t / pix
    float sum = 0.f;
    const int item = tid / pix;
    const long long row = r0 + item;
    if (item < P && row < r_end) {
      const int pp = tid - item * pix;
      const int py = pp / a.Wi, px = pp - py * a.Wi;
      const float* yt = ys + (long long)item * cells * ysw;
      float o[CI];
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) o[ci] = 0.f;
      for (int t = 0; t < ntap; ++t) {
        const int ky = t / a.kw, kx = t - ky * a.kw;
        const int ty = py + a.pad - ky, tx = px + a.pad - kx;
        int q = -1;
        if (ty >= 0 && tx >= 0) {
          if (S1) {
            if (ty <= oy_hi && tx < a.Wo) q = ty * a.Wo + tx;
          } else if (ty % s == 0 && tx % s == 0 && ty / s <= oy_hi && tx / s < a.Wo) {
            q = (ty / s) * a.Wo + tx / s;
          }
        }
        if (q >= 0) {
#pragma unroll
          for (int ci = 0; ci < CI; ++ci) o[ci] += yt[q * ysw + t * CI + ci];
        }
      }
      const long long b = row / a.rows_per_b;
      const long long pz = (row / a.pc) % ((long long)a.pgh * a.pgw);
      const int gy = (int)(pz / a.pgw), gx = (int)(pz - (pz / a.pgw) * a.pgw);
      const int ay = gy * a.psy + a.poy + py, ax = gx * a.psx + a.pox + px;
      if (ay >= 0 && ay < a.img_h && ax >= 0 && ax < a.img_w) {
        const long long dpix = b * a.img_h * a.img_w + (long long)ay * a.img_w + ax;
#pragma unroll
        for (int ci = 0; ci < CI; ++ci) {
          const long long be = dpix * CI + ci;
          const float r = a.radius ? a.radius[be] : a.eps;
          sum += o[ci] * a.center[be] - fabsf(o[ci]) * r;
        }
      }
    }
    contrib[tid] = sum;
    __syncthreads();
    // a wavefront per row sums its pixels' contributions (lane-strided, then a
    // butterfly: a fixed order; one thread over a large window was a serial tail)
    for (int it = wave; it < P; it += WAVES) {
      float tot = 0.f;
      for (int e = lane; e < pix; e += 64) tot += contrib[it * pix + e];
      tot = wave_sum(tot);
      if (lane == 0 && r0 + it < r_end) part[r0 + it] = tot;
    }
    __syncthreads();  // the tap tables and contrib are rewritten by the next group
  }
}

template <int CI, int NB>
void cin_launch(bool s1, unsigned grid, size_t lds, hipStream_t st, const ConvIn& a, int bh, int nbands, int xcd_map,
                int per_wg, long long items, float* part, int P) {
  const dim3 g(grid), b(CIN_THREADS);
  if (per_wg > 1) {
    // footprint windows, P rows at a time (one band each)
    if (s1)
      hipLaunchKernelGGL((conv_input_windows_kernel<CI, NB, true>), g, b, lds, st, a, per_wg, P, items, part);
    else
      hipLaunchKernelGGL((conv_input_windows_kernel<CI, NB, false>), g, b, lds, st, a, per_wg, P, items, part);
  } else if (s1) {
    hipLaunchKernelGGL((conv_input_concretize_kernel<CI, NB, true>), g, b, lds, st, a, bh, nbands, xcd_map, items,
                       part);
  } else {
    hipLaunchKernelGGL((conv_input_concretize_kernel<CI, NB, false>), g, b, lds, st, a, bh, nbands, xcd_map, items,
                       part);
  }
}

hipError_t launch_conv_input_concretize(const ConvIn& a, int rows, float* part, float* rowacc, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (!conv_input_fits(a)) return hipErrorInvalidValue;
  const int bh = cin_band_rows(a);
  const int nb = (a.Hi + bh - 1) / bh;
  if ((long long)rows * nb > 0x7fffffffLL) return hipErrorInvalidValue;
  const int nr = (bh + a.kh - 1 + a.stride - 1) / a.stride + 1;
  const size_t lds = (size_t)nr * a.Wo * cin_row_floats(a.kh * a.kw * a.Ci) * sizeof(float);
  // small footprint windows: several rows per workgroup share its weight
  // registers; whole images: one (row, band) per workgroup, XCD-aware
  const long long items = (long long)rows * nb;
  // (several rows per workgroup need one band of at most 8 M-blocks, whose
  // staged rows are the whole output window)
  const int per_wg = a.patch && nb == 1 && bh == a.Hi && a.Ho * a.Wo <= 128 ? CIN_WIN_ROWS : 1;
  const unsigned grid = (unsigned)((items + per_wg - 1) / per_wg);
  // footprint windows: rows bounded together so that their M-blocks (at most 8)
  // and their input pixels (at most one per thread) fill the workgroup
  int P = 1;
  size_t lds_use = lds;
  if (per_wg > 1) {
    const int mbi = (a.Ho * a.Wo + 15) / 16;
    P = std::max(1, std::min({8 / mbi, CIN_THREADS / (a.Hi * a.Wi), per_wg}));
    lds_use = (size_t)P * a.Ho * a.Wo * cin_row_floats(a.kh * a.kw * a.Ci) * sizeof(float);
  }
  const int xm = per_wg == 1 && rows % 8 == 0;
  const bool s1 = a.stride == 1;
  switch (a.Ci * 4 + cin_col_blocks(a)) {
    case 1 * 4 + 1: cin_launch<1, 1>(s1, grid, lds_use, st, a, bh, nb, xm, per_wg, items, part, P); break;
    case 2 * 4 + 1: cin_launch<2, 1>(s1, grid, lds_use, st, a, bh, nb, xm, per_wg, items, part, P); break;
    case 2 * 4 + 2: cin_launch<2, 2>(s1, grid, lds_use, st, a, bh, nb, xm, per_wg, items, part, P); break;
    case 3 * 4 + 1: cin_launch<3, 1>(s1, grid, lds_use, st, a, bh, nb, xm, per_wg, items, part, P); break;
    case 3 * 4 + 2: cin_launch<3, 2>(s1, grid, lds_use, st, a, bh, nb, xm, per_wg, items, part, P); break;
    case 4 * 4 + 1: cin_launch<4, 1>(s1, grid, lds_use, st, a, bh, nb, xm, per_wg, items, part, P); break;
    case 4 * 4 + 2: cin_launch<4, 2>(s1, grid, lds_use, st, a, bh, nb, xm, per_wg, items, part, P); break;
    case 4 * 4 + 3: cin_launch<4, 3>(s1, grid, lds_use, st, a, bh, nb, xm, per_wg, items, part, P); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rows_reduce(part, 1, rows, nb, 1, 1, rowacc, 1, 0, st);
}

// Identity rows (b, sign, p, c) over a node of P pixels and C channels, on
// each row's own 1 x 1 window: out[row][c'] = sign if c' == c else 0.
__global__ void patch_identity_kernel(long long rows, int R, int C, float* __restrict__ out) {
  const long long total = rows * C;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / C;
    const int cc = (int)(e - row * C);
    const int r = (int)(row % R);
    const float sg = r < R / 2 ? 1.f : -1.f;
    out[e] = (r % C == cc) ? sg : 0.f;
  }
}

// Identity rows (b, sign, p, c) written into a wh x ww window of C channels
// per row: out[row][Y][X][c'] = sign at (cy, cx, c) and 0 elsewhere.
__global__ void window_identity_kernel(long long rows, int R, int C, int wh, int ww, int cy, int cx,
                                       float* __restrict__ out) {
  const int per = wh * ww * C;
  const long long total = rows * per;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / per;
    const int rem = (int)(e - row * per);
    const int cell = rem / C, cc = rem - cell * C;
    const int r = (int)(row % R);
    const float sg = r < R / 2 ? 1.f : -1.f;
    out[e] = (cell == cy * ww + cx && r % C == cc) ? sg : 0.f;
  }
}

hipError_t launch_window_identity(int rows, int R, int C, int wh, int ww, int cy, int cx, float* out,
                                  hipStream_t st) {
  const long long total = (long long)rows * wh * ww * C;
  if (total <= 0) return hipSuccess;
  if (cy < 0 || cy >= wh || cx < 0 || cx >= ww) return hipErrorInvalidValue;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(window_identity_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (long long)rows, R, C, wh,
                     ww, cy, cx, out);
  return hipGetLastError();
}

// A window of sh x sw cells copied into a larger dh x dw window at cell offset
// (oy, ox), zeros elsewhere: dst[row][Y][X][c] = src[row][Y-oy][X-ox][c].
__global__ void window_embed_kernel(const float* __restrict__ src, long long rows, int C, int sh, int sw, int dh,
                                    int dw, int oy, int ox, float* __restrict__ dst) {
  const int per = dh * dw * C;
  const long long total = rows * per;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / per;
    const int rem = (int)(e - row * per);
    const int cell = rem / C, cc = rem - cell * C;
    const int Y = cell / dw - oy, X = cell % dw - ox;
    float v = 0.f;
    if (Y >= 0 && Y < sh && X >= 0 && X < sw) v = src[(row * sh * sw + (long long)Y * sw + X) * C + cc];
    dst[e] = v;
  }
}

hipError_t launch_window_embed(const float* src, int rows, int C, int sh, int sw, int dh, int dw, int oy, int ox,
                               float* dst, hipStream_t st) {
  const long long total = (long long)rows * dh * dw * C;
  if (total <= 0) return hipSuccess;
  if (oy < 0 || ox < 0 || oy + sh > dh || ox + sw > dw) return hipErrorInvalidValue;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(window_embed_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, (long long)rows, C, sh, sw,
                     dh, dw, oy, ox, dst);
  return hipGetLastError();
}

hipError_t launch_patch_identity(int rows, int R, int C, float* out, hipStream_t st) {
  const long long total = (long long)rows * C;
  if (total <= 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(patch_identity_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (long long)rows, R, C, out);
  return hipGetLastError();
}

bool patch_id_relax_fits(const PatchIdRelax& a) { return a.Ci > 0 && a.Co > 0; }

// One wavefront per row; lanes along the row's window, channel fastest, so
// the weight, coefficient and output accesses of a step are contiguous.
__global__ __launch_bounds__(256) void patch_id_relax_kernel(const PatchIdRelax a, int rows,
                                                             float* __restrict__ rowacc) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const long long b = row / a.R;
  const int r = (int)(row - b * a.R);
  const float sg = r < a.R / 2 ? 1.f : -1.f;
  const int c = r % a.Co;
  const int p = (int)((row / a.Co) % ((long long)a.pgh * a.pgw));
  const int py = p / a.pgw, px = p - (p / a.pgw) * a.pgw;
  const int L = a.kh * a.kw * a.Ci;
  const float4* coef = a.coef + b * a.img_h * a.img_w * a.Ci;
  float* out = a.out + row * L;
  float s = 0.f;
  if ((a.Ci & 63) == 0) {
    // channels a multiple of 64: lanes step through each window cell's channels
    // in chunks of 64, the same elements in the same order as the loop below,
    // with no division per element
    int e = lane;
    for (int Y = 0; Y < a.kh; ++Y) {
      const int ay = py * a.psy + a.poy + Y;
      for (int X = 0; X < a.kw; ++X) {
        const int ax = px * a.psx + a.pox + X;
        const bool in = ay >= 0 && ay < a.img_h && ax >= 0 && ax < a.img_w;
        const float* w = a.W + ((long long)(Y * a.kw + X) * a.Co + c) * a.Ci;
        const float4* cp = in ? coef + ((long long)ay * a.img_w + ax) * a.Ci : coef;
        for (int ci = lane; ci < a.Ci; ci += 64, e += 64) {
          const float v = sg * w[ci];
          float o = 0.f;
          if (in) {
            const float4 cf = cp[ci];
            o = v >= 0.f ? v * cf.x : v * cf.y;
            s += (a.bias ? o * a.bias[ci] : 0.f) + fminf(v, 0.f) * cf.z;
          }
          out[e] = o;
        }
      }
    }
    s = wave_sum(s);
    if (lane == 0) rowacc[row] += s;
    return;
  }
  for (int e = lane; e < L; e += 64) {
    const int cell = e / a.Ci, ci = e - cell * a.Ci;
    const int Y = cell / a.kw, X = cell - Y * a.kw;
    const float v = sg * a.W[((long long)cell * a.Co + c) * a.Ci + ci];
    const int ay = py * a.psy + a.poy + Y, ax = px * a.psx + a.pox + X;
    float o = 0.f;
    if (ay >= 0 && ay < a.img_h && ax >= 0 && ax < a.img_w) {
      const float4 cf = coef[((long long)ay * a.img_w + ax) * a.Ci + ci];
      o = v >= 0.f ? v * cf.x : v * cf.y;
      s += (a.bias ? o * a.bias[ci] : 0.f) + fminf(v, 0.f) * cf.z;
    }
    out[e] = o;
  }
  s = wave_sum(s);
  if (lane == 0) rowacc[row] += s;
}

hipError_t launch_patch_id_relax(const PatchIdRelax& a, int rows, float* rowacc, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (!patch_id_relax_fits(a)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(patch_id_relax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a, rows, rowacc);
  return hipGetLastError();
}

__global__ void identity_bias_kernel(int batch, int n, const float* __restrict__ bias, int bias_c,
                                     float* __restrict__ rowacc) {
  const long long total = (long long)batch * 2 * n;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long r = e % (2 * n);
    const float sg = r < n ? 1.f : -1.f;
    const long long i = r < n ? r : r - n;
    rowacc[e] = bias ? sg * bias[i % bias_c] : 0.f;
  }
}

hipError_t launch_identity_bias(int batch, int n, const float* bias, int bias_c, float* rowacc, hipStream_t st) {
  hipLaunchKernelGGL(identity_bias_kernel, dim3(1024), dim3(256), 0, st, batch, n, bias, bias_c > 0 ? bias_c : n,
                     rowacc);
  return hipGetLastError();
}

// +-I rows over an n-wide node: row (b, sign, r) holds sign on column r.
// Workgroups stride over rows, threads along the row (no division per element).
__global__ __launch_bounds__(256) void identity_fill_kernel(int batch, int n, float* __restrict__ lam) {
  const long long rows = (long long)batch * 2 * n;
  for (long long row = blockIdx.x; row < rows; row += gridDim.x) {
    const int r = (int)(row % (2 * n));
    const int col = r < n ? r : r - n;
    const float sg = r < n ? 1.f : -1.f;
    float* out = lam + row * n;
    for (int e = threadIdx.x; e < n; e += 256) out[e] = e == col ? sg : 0.f;
  }
}

hipError_t launch_identity_fill(int batch, int n, float* lam, hipStream_t st) {
  const long long rows = (long long)batch * 2 * n;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(identity_fill_kernel, dim3((unsigned)std::min<long long>(rows, 65536)), dim3(256), 0, st, batch,
                     n, lam);
  return hipGetLastError();
}

// one block (256 threads) per row
__global__ __launch_bounds__(256) void relax_kernel(const float* __restrict__ src, int src_broadcast,
                                                    float scale, const float* __restrict__ addend, int rows,
                                                    int rows_per_b, int P, int N, const float* __restrict__ lo,
                                                    const float* __restrict__ hi,
                                                    const float* __restrict__ bias_z,
                                                    const float* __restrict__ alpha, float* __restrict__ psi_out,
                                                    const int* __restrict__ aidx, int acols,
                                                    float* __restrict__ out, float* __restrict__ rowacc) {
  __shared__ float sh[4];
  const int row = blockIdx.x;
  const long long b = row / rows_per_b;
  const long long L = (long long)P * N;
  float s = 0.f;
  for (long long e = threadIdx.x; e < L; e += 256) {
    const int n = (int)(e % N);
    float v = src_broadcast ? src[(long long)row * N + n] * scale : src[(long long)row * L + e];
    if (addend) v += addend[(long long)row * L + e];
    const float l = lo[b * L + e], u = hi[b * L + e];
    float a, sl, t;
    relax_coeffs(l, u, a, sl, t);
    // per-neuron state: [row][L], or compact [row][acols] at the neuron's column
    const int col = aidx ? aidx[b * L + e] : 0;
    const long long si = aidx ? (long long)row * acols + col : (long long)row * L + e;
    if (alpha && l < 0.f && u > 0.f && col >= 0) a = alpha[si];
    const float o = v >= 0.f ? v * a : v * sl;
    out[(long long)row * L + e] = o;
    if (psi_out && col >= 0) psi_out[si] = v;
    if (bias_z) s += o * bias_z[n];
    s += fminf(v, 0.f) * t;
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) rowacc[row] += s;
}

hipError_t launch_relax(const float* src, int src_broadcast, float scale, const float* addend, int rows,
                        int rows_per_b, int P, int N, const float* lo, const float* hi, const float* bias_z,
                        const float* alpha, float* psi_out, const int* aidx, int acols, float* out, float* rowacc,
                        hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(relax_kernel, dim3(rows), dim3(256), 0, st, src, src_broadcast, scale, addend, rows,
                     rows_per_b, P, N, lo, hi, bias_z, alpha, psi_out, aidx, acols, out, rowacc);
  return hipGetLastError();
}

__global__ void add_kernel(const float* __restrict__ a, const float* __restrict__ b, float sb,
                           float* __restrict__ dst, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    dst[i] = b ? a[i] + sb * b[i] : a[i];
}

hipError_t launch_add(const float* a, const float* b, float sb, float* dst, long long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, b, sb, dst, n);
  return hipGetLastError();
}

__global__ void gap_expand_kernel(const float* __restrict__ src, int rows, int P, int C, float scale,
                                  const float* __restrict__ addend, float* __restrict__ dst) {
  const long long total = (long long)rows * P * C;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    long long r = e / ((long long)P * C);
    int c = (int)(e % C);
    float v = src[r * C + c] * scale;
    if (addend) v += addend[e];
    dst[e] = v;
  }
}

hipError_t launch_gap_expand(const float* src, int rows, int P, int C, float scale, const float* addend,
                             float* dst, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(gap_expand_kernel, dim3(4096), dim3(256), 0, st, src, rows, P, C, scale, addend, dst);
  return hipGetLastError();
}

// one block per row: rowacc[r] (+)= sum A c - |A| r  (+ bias), optional lb/ub
// (any n and alignment).
__global__ __launch_bounds__(256) void concretize_rows_kernel(const float* __restrict__ A, int n, int rows_per_b,
                                                              const float* __restrict__ center,
                                                              const float* __restrict__ radius, float eps,
                                                              const float* __restrict__ lo,
                                                              const float* __restrict__ hi,
                                                              const float* __restrict__ bias, float* lb, float* ub,
                                                              float* rowacc) {
  __shared__ float sh[4];
  const int row = blockIdx.x;
  const long long b = row / rows_per_b;
  float sc = 0.f, sr = 0.f;
  {
    for (int j = threadIdx.x; j < n; j += 256) {
      const float a = A[(long long)row * n + j];
      float c, r;
      if (center) {
        c = center[b * n + j];
        r = radius ? radius[b * n + j] : eps;
      } else {
        const float l = lo[b * n + j], u = hi[b * n + j];
        c = (l + u) * 0.5f;
        r = (u - l) * 0.5f;
      }
      sc += a * c;
      sr += fabsf(a) * r;
    }
  }
  sc = block_sum(sc, sh);
  sr = block_sum(sr, sh);
  if (threadIdx.x == 0) {
    const float bb = bias ? bias[row] : 0.f;
    if (lb) lb[row] = sc - sr + bb;
    if (ub) ub[row] = sc + sr + bb;
    if (rowacc) rowacc[row] += sc - sr;
  }
}

// The same for n % 4 == 0 and 16-byte aligned rows, one wavefront per row (four
// rows per workgroup): a lane issues the non-temporal float4 loads of four
// strides of its row before accumulating (Lambda is read once, so it bypasses
// the caches' retention), the centre / radius come from L2, and the row's sums
// are a fixed-order shuffle tree (no LDS, no barrier).
typedef float cr_v4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void concretize_rows_wave_kernel(const float* __restrict__ A, int n, long long rows,
                                                                   int rows_per_b, const float* __restrict__ center,
                                                                   const float* __restrict__ radius, float eps,
                                                                   const float* __restrict__ lo,
                                                                   const float* __restrict__ hi,
                                                                   const float* __restrict__ bias, float* lb,
                                                                   float* ub, float* rowacc) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wavefront
  const int lane = threadIdx.x & 63;
  const long long b = row / rows_per_b;
  const int n4 = n >> 2;
  const cr_v4* a4 = reinterpret_cast<const cr_v4*>(A + row * n);
  const long long bo = b * n4;
  float sc = 0.f, sr = 0.f;
  for (int j0 = lane; j0 < n4; j0 += 4 * 64) {
    cr_v4 a[4];
    float4 c[4], r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + 64 * u;
      const int jj = j < n4 ? j : j0;
      a[u] = __builtin_nontemporal_load(a4 + jj);
      if (center) {
        c[u] = reinterpret_cast<const float4*>(center)[bo + jj];
        r[u] = radius ? reinterpret_cast<const float4*>(radius)[bo + jj] : make_float4(eps, eps, eps, eps);
      } else {
        const float4 l = reinterpret_cast<const float4*>(lo)[bo + jj];
        const float4 h = reinterpret_cast<const float4*>(hi)[bo + jj];
        c[u] = make_float4((l.x + h.x) * 0.5f, (l.y + h.y) * 0.5f, (l.z + h.z) * 0.5f, (l.w + h.w) * 0.5f);
        r[u] = make_float4((h.x - l.x) * 0.5f, (h.y - l.y) * 0.5f, (h.z - l.z) * 0.5f, (h.w - l.w) * 0.5f);
      }
      if (j >= n4) a[u] = cr_v4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sc += a[u].x * c[u].x + a[u].y * c[u].y + a[u].z * c[u].z + a[u].w * c[u].w;
      sr += fabsf(a[u].x) * r[u].x + fabsf(a[u].y) * r[u].y + fabsf(a[u].z) * r[u].z + fabsf(a[u].w) * r[u].w;
    }
  }
  sc = wave_sum(sc);
  sr = wave_sum(sr);
  if (lane == 0) {
    const float bb = bias ? bias[row] : 0.f;
    if (lb) lb[row] = sc - sr + bb;
    if (ub) ub[row] = sc + sr + bb;
    if (rowacc) rowacc[row] += sc - sr;
  }
}

hipError_t launch_concretize_rows(const float* A, int rows, int n, int rows_per_b, const float* center,
                                  const float* radius, float eps, const float* lo, const float* hi,
                                  const float* bias, float* lb, float* ub, float* rowacc, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  auto al = [](const float* p) { return ((uintptr_t)p & 15) == 0; };
  const bool vec = n % 4 == 0 && al(A) && al(center) && al(radius) && al(lo) && al(hi);
  if (vec)
    hipLaunchKernelGGL(concretize_rows_wave_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, A, n,
                       (long long)rows, rows_per_b, center, radius, eps, lo, hi, bias, lb, ub, rowacc);
  else
    hipLaunchKernelGGL(concretize_rows_kernel, dim3(rows), dim3(256), 0, st, A, n, rows_per_b, center, radius,
                       eps, lo, hi, bias, lb, ub, rowacc);
  return hipGetLastError();
}

__global__ void ibp_eltwise_kernel(int op, const float* __restrict__ lo0, const float* __restrict__ hi0,
                                   const float* __restrict__ lo1, const float* __restrict__ hi1,
                                   float* __restrict__ lo, float* __restrict__ hi, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    if (op == 0) {
      lo[i] = fmaxf(lo0[i], 0.f);
      hi[i] = fmaxf(hi0[i], 0.f);
    } else {
      lo[i] = lo0[i] + lo1[i];
      hi[i] = hi0[i] + hi1[i];
    }
  }
}

hipError_t launch_ibp_eltwise(int op, const float* lo0, const float* hi0, const float* lo1, const float* hi1,
                              float* lo, float* hi, long long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(ibp_eltwise_kernel, dim3((unsigned)blocks), dim3(256), 0, st, op, lo0, hi0, lo1, hi1, lo, hi, n);
  return hipGetLastError();
}

// one thread per (b, c): fixed-order sum over positions, then / P
__global__ void ibp_gap_kernel(const float* __restrict__ lo_in, const float* __restrict__ hi_in, int batch, int P,
                               int C, float* __restrict__ lo, float* __restrict__ hi) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)batch * C) return;
  const long long b = i / C;
  const int c = (int)(i - b * C);
  float sl = 0.f, su = 0.f;
  for (int p = 0; p < P; ++p) {
    sl += lo_in[(b * P + p) * C + c];
    su += hi_in[(b * P + p) * C + c];
  }
  lo[i] = sl / (float)P;
  hi[i] = su / (float)P;
}

hipError_t launch_ibp_gap(const float* lo_in, const float* hi_in, int batch, int P, int C, float* lo, float* hi,
                          hipStream_t st) {
  long long n = (long long)batch * C;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(ibp_gap_kernel, dim3((n + 255) / 256), dim3(256), 0, st, lo_in, hi_in, batch, P, C, lo, hi);
  return hipGetLastError();
}

__global__ void relax_coef_kernel(const float* __restrict__ lo, const float* __restrict__ hi, long long n,
                                  const int* __restrict__ aidx, float4* __restrict__ coef) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const float l = lo[i], u = hi[i];
    float a, s, t;
    relax_coeffs(l, u, a, s, t);
    const int col = (u > 0.f && l < 0.f) ? (aidx ? aidx[i] : 0) : -1;
    coef[i] = make_float4(a, s, t, __int_as_float(col));
  }
}

hipError_t launch_relax_coef(const float* lo, const float* hi, long long n, const int* aidx, float4* coef,
                             hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(relax_coef_kernel, dim3((unsigned)blocks), dim3(256), 0, st, lo, hi, n, aidx, coef);
  return hipGetLastError();
}

__global__ void box_cr_kernel(const float* __restrict__ lo, const float* __restrict__ hi, long long n,
                              float* __restrict__ c, float* __restrict__ r) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x) {
    const float l = lo[i], u = hi[i];
    c[i] = (l + u) * 0.5f;
    r[i] = (u - l) * 0.5f;
  }
}

hipError_t launch_box_center_radius(const float* lo, const float* hi, long long n, float* c, float* r,
                                    hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(box_cr_kernel, dim3((unsigned)blocks), dim3(256), 0, st, lo, hi, n, c, r);
  return hipGetLastError();
}

__global__ void ibp_splitk_kernel(const float* __restrict__ pc, const float* __restrict__ pr, int S, long long MN,
                                  int N, const float* __restrict__ bias, float* __restrict__ lo,
                                  float* __restrict__ hi, float* __restrict__ rlo, float* __restrict__ rhi) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < MN; e += (long long)gridDim.x * blockDim.x) {
    float c = 0.f, r = 0.f;
    for (int q = 0; q < S; ++q) {
      c += pc[q * MN + e];
      r += pr[q * MN + e];
    }
    c += bias ? bias[e % N] : 0.f;
    const float l = c - r, u = c + r;
    lo[e] = l;
    hi[e] = u;
    if (rlo) {
      rlo[e] = fmaxf(l, 0.f);
      rhi[e] = fmaxf(u, 0.f);
    }
  }
}

hipError_t launch_ibp_splitk_finish(const float* pc, const float* pr, int S, long long MN, int N, const float* bias,
                                    float* lo, float* hi, float* rlo, float* rhi, hipStream_t st) {
  if (MN <= 0) return hipSuccess;
  long long blocks = (MN + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(ibp_splitk_kernel, dim3((unsigned)blocks), dim3(256), 0, st, pc, pr, S, MN, N, bias, lo, hi,
                     rlo, rhi);
  return hipGetLastError();
}

// The alpha-CROWN adjoint epilogue of G elements of row m: g[i] is the
// adjoint over z at neuron n[i] (before z's bias, bias[bi[i]]); writes the
// adjoint after the ReLU's relaxation and, on an unstable neuron, takes the
// Adam ascent step on its slope. Elements with ok[i] false are skipped. All
// loads of a stage are issued before any store, so G elements cost one memory
// latency per stage rather than G.
template <int G>
__device__ __forceinline__ void adjoint_coef(const AdjFinish& a, long long bm, const long long (&n)[G],
                                             const bool (&ok)[G], float4 (&cf)[G]) {
#pragma unroll
  for (int i = 0; i < G; ++i) cf[i] = ok[i] ? a.coef[bm + n[i]] : make_float4(0.f, 0.f, 0.f, __int_as_float(-1));
}

// (the same, given the elements' relaxation coefficients from adjoint_coef)
template <int G>
__device__ __forceinline__ void adjoint_elements(const AdjFinish& a, long long m, const long long (&n)[G],
                                                 const int (&bi)[G], const float (&g)[G], const bool (&ok)[G],
                                                 const float4 (&cf)[G]) {
  long long si[G];
  bool uns[G];
  float psi[G], aold[G], am[G], av[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    // per-neuron state, or compact at the coefficient's column of row m (-1: stable, no entry)
    const int col = __float_as_int(cf[i].w);
    si[i] = a.aidx ? m * a.acols + col : m * a.N + n[i];
    uns[i] = col >= 0 && a.alpha_rw != nullptr;
    psi[i] = uns[i] ? a.psi_in[si[i]] : 0.f;
    aold[i] = uns[i] ? a.alpha_rw[si[i]] : 0.f;
    am[i] = uns[i] && a.do_update ? a.adam_m[si[i]] : 0.f;
    av[i] = uns[i] && a.do_update ? a.adam_v[si[i]] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (!ok[i]) continue;
    const float gz = g[i] + (a.bias ? a.bias[bi[i]] : 0.f);
    a.out[m * a.N + n[i]] = !uns[i] ? gz * cf[i].y : (psi[i] >= 0.f ? gz * aold[i] : gz * cf[i].y + cf[i].z);
    if (a.gz_out) a.gz_out[m * a.N + n[i]] = gz;
    if (uns[i] && a.do_update) {
      const float grad = gz * fmaxf(psi[i], 0.f);
      const float mm = a.beta1 * am[i] + (1.f - a.beta1) * grad;
      const float vv = a.beta2 * av[i] + (1.f - a.beta2) * grad * grad;
      a.adam_m[si[i]] = mm;
      a.adam_v[si[i]] = vv;
      const float step = a.lr * (mm * a.bc1) / (sqrtf(vv * a.bc2) + a.adam_eps);
      a.alpha_rw[si[i]] = fminf(fmaxf(aold[i] + step, 0.f), 1.f);
    }
  }
}

__global__ void adjoint_finish_kernel(AdjFinish a) {
  const long long MN = (long long)a.M * a.N;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < MN; e += (long long)gridDim.x * blockDim.x) {
    float g = 0.f;
    for (int q = 0; q < a.S; ++q) g += a.part[q * MN + e];
    const long long m = e / a.N;
    const long long n[1] = {e - m * a.N};
    const int bi[1] = {(int)n[0]};
    const float gg[1] = {g};
    const bool ok[1] = {true};
    float4 cf[1];
    adjoint_coef<1>(a, (m / a.rows_per_b) * a.N, n, ok, cf);
    adjoint_elements<1>(a, m, n, bi, gg, ok, cf);
  }
}

hipError_t launch_adjoint_finish(const AdjFinish& a, hipStream_t st) {
  const long long MN = (long long)a.M * a.N;
  if (MN <= 0) return hipSuccess;
  long long blocks = (MN + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(adjoint_finish_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

namespace {
constexpr int CADJ_THREADS = 256;
constexpr int CADJ_MAXK = 9;               // 4-deep contraction steps: (tap, input channel) pairs <= 36
constexpr int CADJ_SPT = 16;               // staged floats per thread and row: a band's input rows <= 16 KB
constexpr int CADJ_ROWS = 16;              // rows of one input per workgroup (fewer when that leaves CUs idle)
constexpr int CADJ_TLD = 33;               // row stride of a wavefront's 16 x 32 transpose tile in LDS
}  // namespace

// Columns of a row's input image staged with a zero border: pad before, and
// after up to the last pixel the output reaches.
__host__ __device__ inline int cadj_span(int in, int out, int k, int stride, int pad) {
  const int last = (out - 1) * stride - pad + k;  // one past the last input index read
  return pad + (last > in ? last : in);
}
// 16-channel blocks per wavefront: two (32 channels, whole 128-byte lines per
// store) when Co is a multiple of 32, else one.
inline int cadj_nbn(const ConvAdj& c) { return c.Co % 32 == 0 ? 2 : 1; }
// Output pixels per workgroup: the four wavefronts take the channel groups of
// 16-pixel blocks, as many blocks as fill them.
inline int cadj_px(const ConvAdj& c) { return 16 * std::max(1, 4 / (c.Co / (16 * cadj_nbn(c)))); }
// Input rows staged for a band of px output pixels: the output rows the band
// touches (at most (px + Wo - 2) / Wo + 1), their taps included.
inline int cadj_staged(const ConvAdj& c) {
  const int px = cadj_px(c);
  const int orows = std::min(c.Ho, (px + c.Wo - 2) / c.Wo + 1);
  return ((orows - 1) * c.stride + c.kh) * cadj_span(c.Wi, c.Wo, c.kw, c.stride, c.pad) * c.Ci;
}

bool conv_adjoint_fits(const ConvAdj& c) {
  return c.Ci >= 1 && c.Ci <= 4 && c.Co % 16 == 0 && c.Co <= 64 && c.kh * c.kw * c.Ci <= 4 * CADJ_MAXK &&
         c.stride >= 1 && c.pad >= 0 && c.Ho * c.Wo > 0 && cadj_staged(c) <= CADJ_SPT * CADJ_THREADS &&
         (long long)c.Hi * c.Wi * c.Ci <= 0x7fffffffLL;
}

// The adjoint of the alpha-CROWN step through a conv over a few-channel input
// (the first layer), fused with the ReLU's adjoint epilogue: for every output
// pixel p and channel c, g[p][c] = sum over (tap, c_in) of the adjoint over
// the input at the tap's pixel times W[tap][c][c_in], on 16x16x4 fp32 matrix
// blocks (A: output pixel = lane % 16, pair 4j + lane / 16 at step j; B: the
// weights of the same pair for channel 16 * block + lane % 16, in registers),
// then the adjoint epilogue on each result.
//
// A wavefront computes 16 pixels x 16 NBN channels; a workgroup covers px
// output pixels (all Co channels: wavefront w takes channel group w % G of
// 16-pixel block w / G, G = Co / (16 NBN), so each pixel's results are
// written whole by one workgroup) for up to CADJ_ROWS rows of the same input.
// With NBN = 2 the results pass through a wavefront-private transpose tile in
// LDS so that every store instruction writes 32 consecutive channels (whole
// 128-byte lines) of two pixels: stores of 64-byte pieces of lines were
// throttled by the vector L1 (its address unit stalled on it most of the
// time).  The relaxation coefficients of the elements depend on the input
// only: they are read once into registers and serve every row.  The input
// rows the band reaches are staged in LDS with a zero border for all rows at
// once (a step's operand is one offset from the pixel's corner): one wait for
// the loads and one barrier, then the rows run back to back.
template <int CI, int SPT, int NK, int NBN>
__global__ __launch_bounds__(CADJ_THREADS) void conv_adjoint_first_kernel(const ConvAdj c, int nbands, int rchunk,
                                                                         int nchunks, int staged, int tile_off) {
  // [rchunk][staged] band rows [Hb][Wp][CI] per row (later the unstable-element
  // lists), then with NBN = 2 one [16][CADJ_TLD] transpose tile per wavefront at tile_off
  extern __shared__ __attribute__((aligned(16))) float gs[];
  constexpr int E = 4 * NBN;  // results per lane and row
  // workgroup -> (input, chunk of its rows, band of output pixels)
  unsigned n = blockIdx.x;
  const int band = (int)(n % (unsigned)nbands);
  n /= (unsigned)nbands;
  const int chunk = (int)(n % (unsigned)nchunks);
  const long long b = n / (unsigned)nchunks;
  const int rpb = c.a.rows_per_b;
  const long long row0 = b * rpb + (long long)chunk * rchunk;
  const int nr = (int)min((long long)min(rchunk, rpb - chunk * rchunk), (long long)c.a.M - row0);
  if (nr <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, kk = lane >> 4;
  const int G = c.Co / (16 * NBN), PB = max(1, 4 / G), px = 16 * PB;
  const int grp = wave % G, blk = wave / G;
  const bool active = blk < PB;  // (G = 3: the fourth wavefront only stages)
  const int cbase = grp * 16 * NBN;
  const int Wp = cadj_span(c.Wi, c.Wo, c.kw, c.stride, c.pad);
  const int npx = c.Ho * c.Wo;
  const int p0 = band * px, p1 = min(npx, p0 + px);
  const int oy0 = p0 / c.Wo;
  const int r0 = oy0 * c.stride;
  const long long img = (long long)c.Hi * c.Wi * CI;

  // this thread's staged floats (at most SPT): t = tid + 256 i -> (band row,
  // column, channel), as an offset in a row's input image (-1: border or past the end)
  int soff[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int t = tid + CADJ_THREADS * i;
    const int r = t / (Wp * CI), rem = t - r * (Wp * CI);
    const int y = r0 + r - c.pad, x = rem / CI - c.pad, ci = rem - (rem / CI) * CI;
    soff[i] = (t < staged && y >= 0 && y < c.Hi && x >= 0 && x < c.Wi) ? (y * c.Wi + x) * CI + ci : -1;
  }
  // stage every row of the chunk, eight rows' loads in flight at a time (a
  // border slot, or a row past the chunk, loads a valid float and drops it);
  // offsets from the chunk's first row fit 32 bits (rchunk * img < 2^31)
  const float* gsrc = c.g0 + row0 * img;
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int t = tid + CADJ_THREADS * i;
    if (CADJ_THREADS * i >= staged) break;  // (the same for the whole workgroup)
    const int so = soff[i] < 0 ? 0 : soff[i];
    for (int r = 0; r < nr; r += 8) {
      float sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) sv[u] = gsrc[min(r + u, nr - 1) * (int)img + so];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (t < staged && r + u < nr) gs[(r + u) * staged + t] = soff[i] < 0 ? 0.f : sv[u];
    }
  }

  const int ncol = c.kh * c.kw * CI;
  const int nk = (ncol + 3) / 4;  // <= NK
  // per step: this lane's pair as an offset from the pixel's corner, and the weights
  float bw[NK][NBN];
  int off[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int k = 4 * j + kk;
    const bool ok = j < nk && k < ncol;
    const int tap = ok ? k / CI : 0, ci = ok ? k - tap * CI : 0;
    const int ky = tap / c.kw, kx = tap - ky * c.kw;
    off[j] = (ky * Wp + kx) * CI + ci;  // a pair past the last one meets zero weights
#pragma unroll
    for (int nb = 0; nb < NBN; ++nb)
      bw[j][nb] = ok ? c.W[((long long)tap * c.Co + cbase + 16 * nb + li) * CI + ci] : 0.f;
  }

  // This lane's stored results: NBN = 1: pixel pb + 4 kk + i, channel cbase +
  // li (the MFMA layout); NBN = 2: pixel pb + 2 i + lane / 32, channel cbase +
  // lane % 32 (the transposed layout).  Per result: its offset in a row, the
  // factor of the raw adjoint stored in the first pass (the slope of a stable
  // neuron; 1 for an unstable one, finished below) and its state column (-1
  // stable, -2 past the band's end or an idle wavefront: never stored).
  const int pb = p0 + 16 * blk;
  const int sch = cbase + (NBN == 1 ? li : (lane & 31));
  const float bias = c.a.bias ? c.a.bias[sch] : 0.f;
  const float4* coef = c.a.coef + b * (long long)c.a.N;
  const bool have = c.a.alpha_rw != nullptr;  // (a compact layout without unstable neurons has no state at all)
  int eo[E], col[E];
  float fac[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int pp = pb + (NBN == 1 ? 4 * kk + i : 2 * i + (lane >> 5));
    eo[i] = pp * c.Co + sch;
    const float4 cf = active && pp < p1 ? coef[eo[i]] : make_float4(0.f, 0.f, 0.f, __int_as_float(-2));
    col[i] = __float_as_int(cf.w);
    fac[i] = (col[i] >= 0 && have) ? 1.f : cf.y;
  }
  // the A operand's pixel (rows past the band repeat its last pixel)
  const int pa = min(pb + li, p1 - 1);
  const int oya = pa / c.Wo, oxa = pa - oya * c.Wo;
  const int corner = ((oya * c.stride - r0) * Wp + oxa * c.stride) * CI;
  float* tile = gs + tile_off + wave * (16 * CADJ_TLD);

  // Rows back to back: products and the stores of every result (an unstable
  // element's result needs its kept Psi and slope and updates its Adam state:
  // loads whose latency would stall every row, so the row stores the raw
  // adjoint there and the unstable elements of all rows are finished together
  // afterwards).
  __syncthreads();
  if (active) {
    float* orow = c.a.out + row0 * c.a.N;
    float* gzrow = c.a.gz_out ? c.a.gz_out + row0 * c.a.N : nullptr;
    const float* g = gs + corner;
    for (int r = 0; r < nr; ++r) {
      // (all NK operand reads first; steps past nk read offset 0 and meet zero weights)
      float av[NK];
#pragma unroll
      for (int j = 0; j < NK; ++j) av[j] = g[off[j]];
      cin_v4 acc[NBN];
#pragma unroll
      for (int nb = 0; nb < NBN; ++nb) acc[nb] = cin_v4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NK; ++j)
#pragma unroll
        for (int nb = 0; nb < NBN; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bw[j][nb], acc[nb], 0, 0, 0);
      float val[E];
      if (NBN == 1) {
#pragma unroll
        for (int i = 0; i < E; ++i) val[i] = acc[0][i];
      } else {
        // through the tile: element (pixel 4 kk + v, channel 16 nb + li) ->
        // lane (channel lane % 32) slot i (pixel 2 i + lane / 32); the tile
        // is this wavefront's own, whose LDS accesses complete in order
#pragma unroll
        for (int nb = 0; nb < NBN; ++nb)
#pragma unroll
          for (int v = 0; v < 4; ++v) tile[(4 * kk + v) * CADJ_TLD + 16 * nb + li] = acc[nb][v];
#pragma unroll
        for (int i = 0; i < E; ++i) val[i] = tile[(2 * i + (lane >> 5)) * CADJ_TLD + (lane & 31)];
      }
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if (col[i] == -2) continue;
        const float gz = val[i] + bias;
        orow[eo[i]] = gz * fac[i];
        if (gzrow) gzrow[eo[i]] = gz;
      }
      g += staged;
      orow += c.a.N;
      if (gzrow) gzrow += c.a.N;
    }
  }
  if (!have) return;  // (uniform)

  // The unstable elements: each wavefront lists its own (element offset,
  // state column) in LDS, then its lanes take the (row, element) pairs in
  // row-major order, four at a time, all loads first (consecutive lanes:
  // consecutive state columns of one row).
  __syncthreads();  // every wavefront is done with the staged rows
  int2* desc = reinterpret_cast<int2*>(gs) + wave * (64 * E);
  const unsigned long long below = (1ull << lane) - 1ull;
  int nu = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const bool u = col[i] >= 0;
    const unsigned long long m = __ballot(u);
    if (u) desc[nu + __popcll(m & below)] = make_int2(eo[i], col[i]);
    nu += __popcll(m);
  }
  if (nu == 0) return;  // (uniform in the wavefront; no barrier follows)
  // this wavefront's stores of the raw adjoints above are seen by its loads below
  __threadfence_block();
  const int P = nu * nr;
  const bool upd = c.a.do_update;
  for (int q0 = lane; q0 < P; q0 += 4 * 64) {
    float gz[4], psi[4], ao[4], am[4], av[4];
    float4 cf[4];
    long long oi[4], si[4];
    bool okp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = q0 + 64 * k;
      okp[k] = q < P;
      const int r = okp[k] ? q / nu : 0;
      const int2 dd = desc[okp[k] ? q - r * nu : 0];
      const long long row = row0 + r;
      oi[k] = row * c.a.N + dd.x;
      si[k] = c.a.aidx ? row * c.a.acols + dd.y : oi[k];
      cf[k] = coef[dd.x];
      gz[k] = c.a.out[oi[k]];
      psi[k] = c.a.psi_in[si[k]];
      ao[k] = c.a.alpha_rw[si[k]];
      am[k] = upd ? c.a.adam_m[si[k]] : 0.f;
      av[k] = upd ? c.a.adam_v[si[k]] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!okp[k]) continue;
      const float g = gz[k];
      c.a.out[oi[k]] = psi[k] >= 0.f ? g * ao[k] : g * cf[k].y + cf[k].z;
      if (upd) {
        const float grad = g * fmaxf(psi[k], 0.f);
        const float mm = c.a.beta1 * am[k] + (1.f - c.a.beta1) * grad;
        const float vv = c.a.beta2 * av[k] + (1.f - c.a.beta2) * grad * grad;
        c.a.adam_m[si[k]] = mm;
        c.a.adam_v[si[k]] = vv;
        const float step = c.a.lr * (mm * c.a.bc1) / (sqrtf(vv * c.a.bc2) + c.a.adam_eps);
        c.a.alpha_rw[si[k]] = fminf(fmaxf(ao[k] + step, 0.f), 1.f);
      }
    }
  }
}

// (contraction steps: exactly those of a 3x3 kernel, else the most any shape takes)
template <int CI, int NK, int NBN>
void cadj_launch_nk(unsigned grid, size_t lds, hipStream_t st, const ConvAdj& c, int nbands, int rchunk, int nchunks,
                    int staged, int tile_off) {
  if (staged <= 4 * CADJ_THREADS)
    hipLaunchKernelGGL((conv_adjoint_first_kernel<CI, 4, NK, NBN>), dim3(grid), dim3(CADJ_THREADS), lds, st, c,
                       nbands, rchunk, nchunks, staged, tile_off);
  else
    hipLaunchKernelGGL((conv_adjoint_first_kernel<CI, CADJ_SPT, NK, NBN>), dim3(grid), dim3(CADJ_THREADS), lds, st,
                       c, nbands, rchunk, nchunks, staged, tile_off);
}
template <int CI, int NBN>
void cadj_launch(unsigned grid, size_t lds, hipStream_t st, const ConvAdj& c, int nbands, int rchunk, int nchunks,
                 int staged, int tile_off) {
  constexpr int NK3 = (9 * CI + 3) / 4;
  if ((c.kh * c.kw * CI + 3) / 4 <= NK3)
    cadj_launch_nk<CI, NK3, NBN>(grid, lds, st, c, nbands, rchunk, nchunks, staged, tile_off);
  else
    cadj_launch_nk<CI, CADJ_MAXK, NBN>(grid, lds, st, c, nbands, rchunk, nchunks, staged, tile_off);
}
template <int CI>
void cadj_launch_ci(unsigned grid, size_t lds, hipStream_t st, const ConvAdj& c, int nbands, int rchunk, int nchunks,
                    int staged, int tile_off) {
  if (cadj_nbn(c) == 2)
    cadj_launch<CI, 2>(grid, lds, st, c, nbands, rchunk, nchunks, staged, tile_off);
  else
    cadj_launch<CI, 1>(grid, lds, st, c, nbands, rchunk, nchunks, staged, tile_off);
}

hipError_t launch_conv_adjoint_first(const ConvAdj& c, int rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (!conv_adjoint_fits(c) || c.a.M != rows || c.a.N != c.Ho * c.Wo * c.Co || c.a.rows_per_b <= 0)
    return hipErrorInvalidValue;
  const int nbands = (c.Ho * c.Wo + cadj_px(c) - 1) / cadj_px(c);
  const int rpb = c.a.rows_per_b;
  const long long inputs = ((long long)rows + rpb - 1) / rpb;
  // rows of one input per workgroup: CADJ_ROWS, or fewer (down to 3 or 4)
  // while the grid would leave part of the chip without eight workgroups per
  // CU; and at most 40 KB of staged rows
  const int staged = cadj_staged(c);
  int rchunk = std::min(CADJ_ROWS, rpb);
  while (rchunk > 4 && inputs * ((rpb + rchunk - 1) / rchunk) * nbands < 2048) rchunk = (rchunk + 1) / 2;
  rchunk = std::max(1, std::min(rchunk, (int)(40960 / (staged * sizeof(float)))));
  // (the staging addresses a chunk's input rows with 32-bit offsets)
  const long long img = (long long)c.Hi * c.Wi * c.Ci;
  while (rchunk > 1 && rchunk * img > 0x7fffffffLL) rchunk /= 2;
  const int nchunks = (rpb + rchunk - 1) / rchunk;
  const long long grid = inputs * nchunks * nbands;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // LDS: the staged rows, which the unstable-element lists (up to 64 * 4 NBN
  // entries of 8 bytes per wavefront) reuse, then the transpose tiles
  const int nbn = cadj_nbn(c);
  const size_t first = std::max((size_t)rchunk * staged * sizeof(float), (size_t)CADJ_THREADS * 4 * nbn * 8);
  const int tile_off = (int)(first / sizeof(float));
  const size_t lds = first + (nbn == 2 ? (size_t)(CADJ_THREADS / 64) * 16 * CADJ_TLD * sizeof(float) : 0);
  switch (c.Ci) {
    case 1: cadj_launch_ci<1>((unsigned)grid, lds, st, c, nbands, rchunk, nchunks, staged, tile_off); break;
    case 2: cadj_launch_ci<2>((unsigned)grid, lds, st, c, nbands, rchunk, nchunks, staged, tile_off); break;
    case 3: cadj_launch_ci<3>((unsigned)grid, lds, st, c, nbands, rchunk, nchunks, staged, tile_off); break;
    default: cadj_launch_ci<4>((unsigned)grid, lds, st, c, nbands, rchunk, nchunks, staged, tile_off); break;
  }
  return hipGetLastError();
}

// one thread per output element of the im2col image (coalesced writes)
__global__ void im2col_kernel(const float* __restrict__ src, int rows, int H, int W, int C, int kh, int kw,
                              int stride, int pad, int Ho, int Wo, int Kp, float* __restrict__ dst) {
  const long long total = (long long)rows * Ho * Wo * Kp;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long long)gridDim.x * blockDim.x) {
    const int k = (int)(e % Kp);
    const long long p = e / Kp;  // (row, oy, ox)
    const int ox = (int)(p % Wo);
    const long long t = p / Wo;
    const int oy = (int)(t % Ho);
    const long long row = t / Ho;
    float v = 0.f;
    if (k < kh * kw * C) {
      const int tap = k / C, c = k - tap * C;
      const int y = oy * stride - pad + tap / kw, x = ox * stride - pad + tap % kw;
      if (y >= 0 && y < H && x >= 0 && x < W) v = src[((row * H + y) * W + x) * C + c];
    }
    dst[e] = v;
  }
}

hipError_t launch_im2col(const float* src, int rows, int H, int W, int C, int kh, int kw, int stride, int pad,
                         int Ho, int Wo, int Kp, float* dst, hipStream_t st) {
  const long long total = (long long)rows * Ho * Wo * Kp;
  if (total <= 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(im2col_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, rows, H, W, C, kh, kw, stride,
                     pad, Ho, Wo, Kp, dst);
  return hipGetLastError();
}

__global__ void pad_weights_kernel(const float* __restrict__ Wt, int taps, int N, int C, int Kp,
                                   float* __restrict__ dst) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N * Kp) return;
  const int n = e / Kp, k = e - n * Kp;
  float v = 0.f;
  if (k < taps * C) {
    const int tap = k / C, c = k - tap * C;
    v = Wt[((long long)tap * N + n) * C + c];
  }
  dst[e] = v;
}

hipError_t launch_pad_weights(const float* W, int taps, int N, int C, int Kp, float* dst, hipStream_t st) {
  if (N * Kp <= 0) return hipSuccess;
  hipLaunchKernelGGL(pad_weights_kernel, dim3((N * Kp + 255) / 256), dim3(256), 0, st, W, taps, N, C, Kp, dst);
  return hipGetLastError();
}

__global__ void fill_kernel(float* p, float v, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill(float* p, float v, long long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

__global__ void alpha_init_kernel(const float* __restrict__ lo, const float* __restrict__ hi, int batch,
                                  int rows_per_b, long long n, float* __restrict__ alpha,
                                  float* __restrict__ am, float* __restrict__ av) {
  const long long total = (long long)batch * rows_per_b * n;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / n, j = e - row * n;
    const long long b = row / rows_per_b;
    const float l = lo[b * n + j], u = hi[b * n + j];
    float a, s, t;
    relax_coeffs(l, u, a, s, t);
    alpha[e] = a;
    am[e] = 0.f;
    av[e] = 0.f;
  }
}

// Compact state: one thread per (b, neuron); an unstable neuron writes its
// column of the rows_per_b rows of b.
__global__ void alpha_init_compact_kernel(const float* __restrict__ lo, const float* __restrict__ hi, int batch,
                                          int rows_per_b, long long n, const int* __restrict__ aidx, int acols,
                                          float* __restrict__ alpha, float* __restrict__ am, float* __restrict__ av) {
  const long long total = (long long)batch * n;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const int col = aidx[e];
    if (col < 0) continue;
    const long long b = e / n;
    float a, s, t;
    relax_coeffs(lo[e], hi[e], a, s, t);
    for (int r = 0; r < rows_per_b; ++r) {
      const long long o = (b * rows_per_b + r) * acols + col;
      alpha[o] = a;
      am[o] = 0.f;
      av[o] = 0.f;
    }
  }
}

hipError_t launch_alpha_init(const float* lo, const float* hi, int batch, int rows_per_b, long long n,
                             const int* aidx, int acols, float* alpha, float* am, float* av, hipStream_t st) {
  if (batch <= 0 || n <= 0) return hipSuccess;
  if (aidx) {
    if (acols <= 0) return hipSuccess;  // no unstable neuron: no state
    hipLaunchKernelGGL(alpha_init_compact_kernel, dim3(2048), dim3(256), 0, st, lo, hi, batch, rows_per_b, n, aidx,
                       acols, alpha, am, av);
  } else {
    hipLaunchKernelGGL(alpha_init_kernel, dim3(4096), dim3(256), 0, st, lo, hi, batch, rows_per_b, n, alpha, am, av);
  }
  return hipGetLastError();
}

// Column of every unstable neuron of batch element blockIdx.x: an exclusive
// scan of the 0/1 unstable flags in node order, 256 neurons per pass (wave
// ballots, then the four wave totals in LDS).
__global__ __launch_bounds__(256) void alpha_layout_kernel(const float* __restrict__ lo, const float* __restrict__ hi,
                                                           long long n, int* __restrict__ idx,
                                                           int* __restrict__ count) {
  __shared__ int wsum[4];
  const long long b = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int base = 0;
  for (long long j0 = 0; j0 < n; j0 += 256) {
    const long long j = j0 + threadIdx.x;
    bool uns = false;
    if (j < n) {
      const float l = lo[b * n + j], u = hi[b * n + j];
      uns = l < 0.f && u > 0.f;
    }
    const unsigned long long mask = __ballot(uns);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(mask);
    __syncthreads();
    int off = base;
    for (int q = 0; q < w; ++q) off += wsum[q];
    if (j < n) idx[b * n + j] = uns ? off + before : -1;
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) count[b] = base;
}

hipError_t launch_alpha_layout(const float* lo, const float* hi, int batch, long long n, int* idx, int* count,
                               hipStream_t st) {
  if (batch <= 0 || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(alpha_layout_kernel, dim3((unsigned)batch), dim3(256), 0, st, lo, hi, n, idx, count);
  return hipGetLastError();
}

__global__ void adj_domain_kernel(const float* __restrict__ psi, int rows, int n, int rows_per_b,
                                  const float* __restrict__ center, const float* __restrict__ radius, float eps,
                                  float* __restrict__ g) {
  const long long total = (long long)rows * n;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / n, j = e - row * n;
    const long long bj = (row / rows_per_b) * n + j;
    const float p = psi[e];
    const float r = radius ? radius[bj] : eps;
    const float sg = p > 0.f ? 1.f : (p < 0.f ? -1.f : 0.f);
    g[e] = center[bj] - r * sg;
  }
}

hipError_t launch_adj_domain(const float* psi, int rows, int n, int rows_per_b, const float* center,
                             const float* radius, float eps, float* g, hipStream_t st) {
  if (rows <= 0 || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(adj_domain_kernel, dim3(2048), dim3(256), 0, st, psi, rows, n, rows_per_b, center, radius, eps,
                     g);
  return hipGetLastError();
}

// dst[b][c][r] = src[b][r][c] for b < batch (32x32 LDS tiles)
__global__ __launch_bounds__(256) void transpose_kernel(const float* __restrict__ src, int R, int C,
                                                        float* __restrict__ dst) {
  __shared__ float t[32][33];
  const long long boff = (long long)blockIdx.z * R * C;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int y = ty; y < 32; y += 8) {
    const int r = r0 + y, c = c0 + tx;
    if (r < R && c < C) t[y][tx] = src[boff + (long long)r * C + c];
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int c = c0 + y, r = r0 + tx;
    if (r < R && c < C) dst[boff + (long long)c * R + r] = t[tx][y];
  }
}

hipError_t launch_transpose(const float* src, int batch, int R, int C, float* dst, hipStream_t st) {
  if (batch <= 0 || R <= 0 || C <= 0) return hipSuccess;
  dim3 g((C + 31) / 32, (R + 31) / 32, batch);
  hipLaunchKernelGGL(transpose_kernel, g, dim3(256), 0, st, src, R, C, dst);
  return hipGetLastError();
}

// Verdict per input: verified[b] = 1 iff lb[b][i] > 0 for every spec i (a NaN
// bound is not > 0); one workgroup per input.
__global__ __launch_bounds__(256) void verify_kernel(const float* __restrict__ lb, int m,
                                                     int* __restrict__ verified) {
  const int b = blockIdx.x;
  int ok = 1;
  for (int i = threadIdx.x; i < m; i += blockDim.x) ok &= (lb[(long long)b * m + i] > 0.f) ? 1 : 0;
  ok = __syncthreads_and(ok);
  if (threadIdx.x == 0) verified[b] = ok;
}

// count[0] = sum of flags[0..n) (one workgroup, fixed order of the partial sums)
__global__ __launch_bounds__(256) void count_kernel(const int* __restrict__ flags, int n, int* __restrict__ count) {
  __shared__ int part[256];
  int s = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s += flags[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) count[0] = part[0];
}

hipError_t launch_verify(const float* lb, int batch, int m, int* verified, int* count, hipStream_t st) {
  hipLaunchKernelGGL(verify_kernel, dim3(batch), dim3(256), 0, st, lb, m, verified);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !count) return e;
  hipLaunchKernelGGL(count_kernel, dim3(1), dim3(256), 0, st, verified, batch, count);
  return hipGetLastError();
}

// ---- beta-CROWN: split constraints of branch-and-bound sub-domains

// lo = max(lo, 0) where split > 0, hi = min(hi, 0) where split < 0 (n elements)
__global__ void apply_splits_kernel(const float* __restrict__ split, long long n, float* __restrict__ lo,
                                    float* __restrict__ hi) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (long long)gridDim.x * blockDim.x) {
    const float s = split[e];
    if (s > 0.f) lo[e] = fmaxf(lo[e], 0.f);
    if (s < 0.f) hi[e] = fminf(hi[e], 0.f);
  }
}

hipError_t launch_apply_splits(const float* split, long long n, float* lo, float* hi, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(apply_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, st, split, n, lo, hi);
  return hipGetLastError();
}

// Lambda over a split ReLU input: lam[row][j] -= beta[row][j] * split[b][j] and
// rowacc[row] += sum_j (-beta * split)[j] * bias[j % bias_c]; one wavefront per row.
__global__ __launch_bounds__(256) void beta_apply_kernel(float* __restrict__ lam, int rows, int R, int n,
                                                         const float* __restrict__ beta,
                                                         const float* __restrict__ split,
                                                         const float* __restrict__ bias, int bias_c,
                                                         float* __restrict__ rowacc) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const long long b = row / R;
  const float* sp = split + b * n;
  float* l = lam + row * n;
  const float* be = beta + row * n;
  float acc = 0.f;
  for (int j = lane; j < n; j += 64) {
    const float sg = sp[j];
    if (sg != 0.f) {
      const float d = -be[j] * sg;
      l[j] += d;
      if (bias) acc += d * bias[bias_c > 0 ? j % bias_c : j];
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) rowacc[row] += acc;
}

hipError_t launch_beta_apply(float* lam, int rows, int R, int n, const float* beta, const float* split,
                             const float* bias, int bias_c, float* rowacc, hipStream_t st) {
  if (rows <= 0 || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(beta_apply_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, lam, rows, R, n, beta,
                     split, bias, bias_c, rowacc);
  return hipGetLastError();
}

// Projected Adam ascent on the multipliers of split neurons: d(sum lb)/d beta =
// -split * gz (gz: the adjoint over the ReLU input); beta = max(0, beta + step).
__global__ void beta_adam_kernel(long long total, int R, int n, const float* __restrict__ gz,
                                 const float* __restrict__ split, float* __restrict__ beta, float* __restrict__ bm,
                                 float* __restrict__ bv, float lr, float b1, float b2, float bc1, float bc2,
                                 float eps) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long row = e / n;
    const int j = (int)(e - row * n);
    const float sg = split[(row / R) * n + j];
    if (sg == 0.f) continue;
    const float grad = -sg * gz[e];
    const float mm = b1 * bm[e] + (1.f - b1) * grad;
    const float vv = b2 * bv[e] + (1.f - b2) * grad * grad;
    bm[e] = mm;
    bv[e] = vv;
    const float step = lr * (mm * bc1) / (sqrtf(vv * bc2) + eps);
    beta[e] = fmaxf(beta[e] + step, 0.f);
  }
}

hipError_t launch_beta_adam(int rows, int R, int n, const float* gz, const float* split, float* beta, float* bm,
                            float* bv, float lr, float b1, float b2, float bc1, float bc2, float eps,
                            hipStream_t st) {
  const long long total = (long long)rows * n;
  if (total <= 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(beta_adam_kernel, dim3((unsigned)blocks), dim3(256), 0, st, total, R, n, gz, split, beta, bm,
                     bv, lr, b1, b2, bc1, bc2, eps);
  return hipGetLastError();
}

// Branching score of every neuron of a ReLU input, per sub-domain b:
// score[b][j] = sum over rows r of b with best[b][r] <= 0 of max(-psi[b*R + r][j], 0) * t_j,
// t = -u l / (u - l) on unstable neurons (l < 0 < u); -inf on stable neurons.
__global__ void branch_score_kernel(const float* __restrict__ psi, const float* __restrict__ best, int batch, int R,
                                    int n, const float* __restrict__ lo, const float* __restrict__ hi,
                                    float* __restrict__ score) {
  const long long total = (long long)batch * n;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const long long b = e / n;
    const int j = (int)(e - b * n);
    const float l = lo[e], u = hi[e];
    if (!(l < 0.f && u > 0.f)) {
      score[e] = -INFINITY;
      continue;
    }
    const float t = -u * l / (u - l);
    float sc = 0.f;
    for (int r = 0; r < R; ++r) {
      if (best[b * R + r] > 0.f) continue;
      sc += fmaxf(-psi[(b * R + r) * n + j], 0.f) * t;
    }
    score[e] = sc;
  }
}

hipError_t launch_branch_score(const float* psi, const float* best, int batch, int R, int n, const float* lo,
                               const float* hi, float* score, hipStream_t st) {
  const long long total = (long long)batch * n;
  if (total <= 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(branch_score_kernel, dim3((unsigned)blocks), dim3(256), 0, st, psi, best, batch, R, n, lo, hi,
                     score);
  return hipGetLastError();
}

// dst[b][e] = src[e] for b < batch (n elements per copy)
__global__ void broadcast_kernel(const float* __restrict__ src, long long n, int batch, float* __restrict__ dst) {
  const long long total = n * batch;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long long)gridDim.x * blockDim.x)
    dst[e] = src[e % n];
}

hipError_t launch_broadcast(const float* src, long long n, int batch, float* dst, hipStream_t st) {
  const long long total = n * batch;
  if (total <= 0) return hipSuccess;
  long long blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(broadcast_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, n, batch, dst);
  return hipGetLastError();
}

}  // namespace vb

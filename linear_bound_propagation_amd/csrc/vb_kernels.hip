// HIP kernels for CDNA4 (gfx950) linear bound propagation.
//
// The hot operation of CROWN back-substitution (the A matrices of "Scaling
// Neural Network Verification with Tensor Parallelism and Fully Sharded Data
// Parallelism", Sec. 1 and Sec. 4.1) is Psi = Lambda W for Linear nodes and
// Psi = conv^T(Lambda, W) for Conv nodes, followed by the ReLU relaxation with
// slopes from intermediate bounds (Sec. 2.1).  Both are one implicit GEMM here:
// an output position gathers its A row from up to 9 shifted positions of a
// channels-last source (one "tap" each), and the reduction runs over
// (tap, channel).  A plain GEMM is the one-tap, one-position case.  The GEMM
// runs on fp32 MFMA (v_mfma_f32_32x32x2f32, 64-wide wavefronts) with LDS
// double-buffered tiles; the relaxation, the concretisation over the domain
// box and the IBP interval arithmetic are fused into its epilogue, which also
// reduces each output row to a per-tile partial sum (no float atomics: the
// partials are summed later in a fixed order, so results are deterministic).
#include <hip/hip_runtime.h>

#include "vb_internal.h"

namespace vb {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NTHR = 256;  // 4 wavefronts of 64
constexpr int BK = 16;     // reduction depth per LDS stage
constexpr int PAD = 4;     // LDS row padding (floats)

// ---------------------------------------------------------------------------
// implicit GEMM

struct PosInfo {
  long long a_base;  // A offset of (row) for gathers, or of the row for dense
  int Y, X;
  bool valid;
};

template <bool DENSE>
__device__ __forceinline__ PosInfo pos_info(const GemmDesc& d, int m) {
  PosInfo p;
  p.valid = m < d.M;
  int mm = p.valid ? m : 0;
  if (DENSE) {
    p.a_base = (long long)mm * d.a_row_stride;
    p.Y = 0;
    p.X = 0;
  } else {
    int P = d.gh * d.gw;
    int row = mm / P;
    int q = mm - row * P;
    p.Y = q / d.gw;
    p.X = q - p.Y * d.gw;
    p.a_base = (long long)row * d.a_row_stride;
  }
  return p;
}

// Offset of A element (position p, reduction index k) or -1 when it is padding.
template <bool DENSE>
__device__ __forceinline__ long long a_offset(const GemmDesc& d, const PosInfo& p, int k) {
  if (!p.valid || k >= d.K) return -1;
  if (DENSE) return p.a_base + k;
  int j = (d.ntaps == 1) ? 0 : k / d.cs;
  int c = k - j * d.cs;
  int yy = p.Y * d.sy + d.tap_dy[j];
  int xx = p.X * d.sx + d.tap_dx[j];
  if (yy < 0 || yy >= d.hs || xx < 0 || xx >= d.ws) return -1;
  return p.a_base + ((long long)yy * d.ws + xx) * d.cs + c;
}

__device__ __forceinline__ long long b_offset(const GemmDesc& d, int k, int n) {
  if (k >= d.K || n >= d.N) return -1;
  int j = (d.ntaps == 1) ? 0 : k / d.cs;
  int c = k - j * d.cs;
  int t = d.tap_w[j];
  if (!d.btrans) return ((long long)t * d.cs + c) * d.N + n;
  return ((long long)t * d.N + n) * d.cs + c;
}

template <int AMODE>
__device__ __forceinline__ void a_value(const GemmDesc& d, long long off, float& c, float& r) {
  if (off < 0) {
    c = 0.f;
    r = 0.f;
    return;
  }
  if (AMODE == A_PLAIN) {
    c = d.A[off];
    r = 0.f;
  } else if (AMODE == A_IBP_BOX) {
    float l = d.A[off], u = d.A2[off];
    c = (l + u) * 0.5f;
    r = (u - l) * 0.5f;
  } else {
    c = d.A[off];
    r = d.A2 ? d.A2[off] : d.eps;
  }
}

template <int BM, int BN, int WM, int WN, bool DENSE, int AMODE, int EPI>
__global__ __launch_bounds__(NTHR) void gemm_kernel(const GemmDesc d) {
  constexpr int NA = (AMODE == A_PLAIN) ? 1 : 2;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_PER = BM * BK / NTHR;          // A scalars per thread per stage
  constexpr int B_PER = (BN * BK + NTHR - 1) / NTHR;
  static_assert(WM * WN == NTHR / 64, "4 waves");
  static_assert(FM >= 1 && FN >= 1, "wave tile");

  __shared__ float As[2][NA][BK][BM + PAD];
  __shared__ float Bs[2][BK][BN + PAD];
  __shared__ float red[WN][BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // XCD-aware tile order: workgroups are dispatched round-robin over the 8
  // XCDs, so give each XCD a contiguous run of tiles, N-tiles of one M-tile
  // adjacent, and the A rows of an M-tile stay in that XCD's L2.
  const int mt = (d.M + BM - 1) / BM;
  const int nt = (d.N + BN - 1) / BN;
  const int total = mt * nt;
  const int per_xcd = (total + 7) / 8;
  const int bid = blockIdx.x;
  const int tile = (bid & 7) * per_xcd + (bid >> 3);
  if (tile >= total) return;
  const int tm = tile / nt, tn = tile - (tile / nt) * nt;
  const int m0 = tm * BM, n0 = tn * BN;

  // A: element e = tid + NTHR*i of the BM x BK stage, row = e / BK, kk = e % BK
  // (consecutive threads walk along k of one row; four rows per wavefront)
  PosInfo pinf[A_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    int e = tid + NTHR * i;
    pinf[i] = pos_info<DENSE>(d, m0 + e / BK);
  }

  float ra[NA][A_PER];
  float rb[B_PER];

  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      int e = tid + NTHR * i;
      long long off = a_offset<DENSE>(d, pinf[i], k0 + (e % BK));
      float c, r;
      a_value<AMODE>(d, off, c, r);
      ra[0][i] = c;
      if (NA == 2) ra[NA - 1][i] = r;
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      int e = tid + NTHR * i;
      float v = 0.f;
      if (e < BN * BK) {
        int k, n;
        if (d.btrans) {  // contiguous along k: consecutive threads walk k
          n = e / BK;
          k = e % BK;
        } else {         // contiguous along n
          k = e / BN;
          n = e % BN;
        }
        long long off = b_offset(d, k0 + k, n0 + n);
        if (off >= 0) v = d.B[off];
      }
      rb[i] = v;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      int e = tid + NTHR * i;
      As[buf][0][e % BK][e / BK] = ra[0][i];
      if (NA == 2) As[buf][NA - 1][e % BK][e / BK] = ra[NA - 1][i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      int e = tid + NTHR * i;
      if (e < BN * BK) {
        if (d.btrans)
          Bs[buf][e % BK][e / BK] = rb[i];
        else
          Bs[buf][e / BN][e % BN] = rb[i];
      }
    }
  };

  f32x16 acc[FM][FN];
  f32x16 accr[(AMODE == A_PLAIN) ? 1 : FM][(AMODE == A_PLAIN) ? 1 : FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    }
  if (AMODE != A_PLAIN) {
#pragma unroll
    for (int i = 0; i < ((AMODE == A_PLAIN) ? 1 : FM); ++i)
#pragma unroll
      for (int j = 0; j < ((AMODE == A_PLAIN) ? 1 : FN); ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) accr[i][j][v] = 0.f;
  }

  const int nk = (d.K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  const int l32 = lane & 31;
  const int khalf = lane >> 5;
  for (int t = 0; t < nk; ++t) {
    const int cur = t & 1;
    if (t + 1 < nk) load_stage((t + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
      const int k = 2 * kk + khalf;
      float a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = As[cur][0][k][wm * WTM + i * 32 + l32];
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = Bs[cur][k][wn * WTN + j * 32 + l32];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
      if (AMODE != A_PLAIN) {
        float ar[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) ar[i] = As[cur][NA - 1][k][wm * WTM + i * 32 + l32];
#pragma unroll
        for (int i = 0; i < ((AMODE == A_PLAIN) ? 1 : FM); ++i)
#pragma unroll
          for (int j = 0; j < ((AMODE == A_PLAIN) ? 1 : FN); ++j)
            accr[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[i], fabsf(b[j]), accr[i][j], 0, 0, 0);
      }
    }
    if (t + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Lane layout of a 32x32 fp32 MFMA result: register v of
  // lane l holds row 8*(v/4) + 4*(l/32) + v%4, column l%32.
  constexpr bool ROWSUM = (EPI != E_IBP);
  const bool do_rows = ROWSUM && (d.part != nullptr);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int lr = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
      const int m = m0 + lr;
      float rowsum = 0.f;
      if (m < d.M) {
        long long opos, bpos;
        if (DENSE) {
          opos = m;
          bpos = m / d.rows_per_b;
        } else {
          int P = d.gh * d.gw;
          int row = m / P;
          int q = m - row * P;
          int Y = q / d.gw;
          int X = q - Y * d.gw;
          int oy = Y * d.oym + d.oy0, ox = X * d.oxm + d.ox0;
          long long sp = (long long)oy * d.wo + ox;
          opos = (long long)row * d.ho * d.wo + sp;
          bpos = (long long)(row / d.rows_per_b) * d.ho * d.wo + sp;
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = n0 + wn * WTN + j * 32 + l32;
          if (n < d.N) {
            const long long oi = opos * d.N + n;
            const long long bi = bpos * d.N + n;
            float val = acc[i][j][v];
            if (EPI == E_IBP) {
              float cc = val + (d.bias ? d.bias[n] : 0.f);
              float rr = accr[(AMODE == A_PLAIN) ? 0 : i][(AMODE == A_PLAIN) ? 0 : j][v];
              float l = cc - rr, u = cc + rr;
              d.out[oi] = l;
              d.out2[oi] = u;
              if (d.relu_lo) {
                d.relu_lo[oi] = fmaxf(l, 0.f);
                d.relu_hi[oi] = fmaxf(u, 0.f);
              }
            } else {
              if (d.addend) val += d.addend[oi];
              if (EPI == E_STORE) {
                d.out[oi] = val;
                if (d.bias) rowsum += val * d.bias[n];
              } else if (EPI == E_RELAX) {
                const float l = d.lo[bi], u = d.hi[bi];
                float a, s, tt;
                if (u <= 0.f) {
                  a = 0.f; s = 0.f; tt = 0.f;
                } else if (l >= 0.f) {
                  a = 1.f; s = 1.f; tt = 0.f;
                } else {
                  s = u / (u - l);
                  tt = -s * l;
                  a = d.alpha ? d.alpha[oi] : ((u >= -l) ? 1.f : 0.f);
                }
                const float o = (val >= 0.f) ? val * a : val * s;
                d.out[oi] = o;
                if (d.psi_out) d.psi_out[oi] = val;
                if (d.bias) rowsum += o * d.bias[n];
                rowsum += fminf(val, 0.f) * tt;
              } else {  // E_CONCRETIZE
                float c, r;
                if (d.center) {
                  c = d.center[bi];
                  r = d.radius ? d.radius[bi] : d.eps;
                } else {
                  const float l = d.lo[bi], u = d.hi[bi];
                  c = (l + u) * 0.5f;
                  r = (u - l) * 0.5f;
                }
                rowsum += val * c - fabsf(val) * r;
              }
            }
          }
        }
      }
      if (ROWSUM) {
        // sum over the 32 columns held by the 32 lanes of this half-wavefront
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) rowsum += __shfl_xor(rowsum, o, 32);
        if (l32 == 0) red[wn][lr] = rowsum;
      }
    }
  }
  if (ROWSUM) {
    __syncthreads();
    if (do_rows) {
      for (int r = tid; r < BM; r += NTHR) {
        const int m = m0 + r;
        if (m < d.M) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < WN; ++w) s += red[w][r];
          d.part[(long long)m * d.part_ld + tn] = s;
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool DENSE>
static hipError_t launch_cfg(const GemmDesc& d, hipStream_t st) {
  const int mt = (d.M + BM - 1) / BM;
  const int nt = (d.N + BN - 1) / BN;
  const int total = mt * nt;
  const int grid = ((total + 7) / 8) * 8;
  dim3 g(grid), b(NTHR);
  switch (d.epi) {
    case E_STORE:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_STORE>), g, b, 0, st, d);
      break;
    case E_RELAX:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_RELAX>), g, b, 0, st, d);
      break;
    case E_CONCRETIZE:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_CONCRETIZE>), g, b, 0, st, d);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool DENSE>
static hipError_t launch_ibp_cfg(const GemmDesc& d, int amode, hipStream_t st) {
  const int mt = (d.M + BM - 1) / BM;
  const int nt = (d.N + BN - 1) / BN;
  const int grid = ((mt * nt + 7) / 8) * 8;
  dim3 g(grid), b(NTHR);
  if (amode == A_IBP_BOX)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_IBP_BOX, E_IBP>), g, b, 0, st, d);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_IBP_BALL, E_IBP>), g, b, 0, st, d);
  return hipGetLastError();
}

static int tile_n(int N) { return N > 64 ? 128 : (N > 32 ? 64 : 32); }

int gemm_ntiles(const GemmDesc& d) {
  const int bn = tile_n(d.N);
  return (d.N + bn - 1) / bn;
}

static bool is_dense(const GemmDesc& d) {
  return d.gh == 1 && d.gw == 1 && d.hs == 1 && d.ws == 1 && d.ntaps == 1 && d.cs == d.K &&
         d.tap_dy[0] == 0 && d.tap_dx[0] == 0 && d.tap_w[0] == 0 && d.ho == 1 && d.wo == 1;
}

hipError_t launch_gemm(const GemmDesc& d, hipStream_t st) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  const bool dense = is_dense(d);
  const int bn = tile_n(d.N);
  if (d.epi == E_IBP) {
    const int amode = d.amode;
    if (bn == 128)
      return dense ? launch_ibp_cfg<128, 128, 2, 2, true>(d, amode, st)
                   : launch_ibp_cfg<128, 128, 2, 2, false>(d, amode, st);
    if (bn == 64)
      return dense ? launch_ibp_cfg<256, 64, 4, 1, true>(d, amode, st)
                   : launch_ibp_cfg<256, 64, 4, 1, false>(d, amode, st);
    return dense ? launch_ibp_cfg<256, 32, 4, 1, true>(d, amode, st)
                 : launch_ibp_cfg<256, 32, 4, 1, false>(d, amode, st);
  }
  if (bn == 128)
    return dense ? launch_cfg<128, 128, 2, 2, true>(d, st) : launch_cfg<128, 128, 2, 2, false>(d, st);
  if (bn == 64)
    return dense ? launch_cfg<256, 64, 4, 1, true>(d, st) : launch_cfg<256, 64, 4, 1, false>(d, st);
  return dense ? launch_cfg<256, 32, 4, 1, true>(d, st) : launch_cfg<256, 32, 4, 1, false>(d, st);
}

// ---------------------------------------------------------------------------
// reductions and elementwise kernels

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
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
                                                          int accumulate) {
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
    s += part[(((long long)z * rows + row) * P + p) * ld + c];
  }
  s = wave_sum(s);
  if (lane == 0) rowacc[row] = accumulate ? rowacc[row] + s : s;
}

hipError_t launch_rows_reduce(const float* part, int Z, int rows, int P, int S, int ld, float* rowacc,
                              int accumulate, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rows_reduce_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, part, Z, rows, P, S, ld,
                     rowacc, accumulate);
  return hipGetLastError();
}

__global__ void finish_kernel(const float* __restrict__ acc, int batch, int R, float* lb, float* ub,
                              float* best) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)batch * R) return;
  const long long b = i / R, r = i - b * R;
  const float l = acc[b * 2 * R + r];
  if (lb) lb[i] = l;
  if (ub) ub[i] = -acc[b * 2 * R + R + r];
  if (best) best[i] = fmaxf(best[i], l);
}

hipError_t launch_finish(const float* rowacc, int batch, int R, float* lb, float* ub, float* best,
                         hipStream_t st) {
  long long n = (long long)batch * R;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(finish_kernel, dim3((n + 255) / 256), dim3(256), 0, st, rowacc, batch, R, lb, ub, best);
  return hipGetLastError();
}

// one wave per spec row
__global__ __launch_bounds__(256) void spec_init_kernel(const float* __restrict__ C, int batch, int m, int n,
                                                        const float* __restrict__ bias, float* __restrict__ lam,
                                                        float* __restrict__ rowacc, int split) {
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
    if (bias) s += v * bias[j];
  }
  s = wave_sum(s);
  if (lane == 0) rowacc[row] = s;
}

hipError_t launch_spec_init(const float* C, int batch, int m, int n, const float* bias, float* lam,
                            float* rowacc, int split, hipStream_t st) {
  long long rows = (long long)batch * (split ? 2 * m : m);
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(spec_init_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, C, batch, m, n, bias, lam,
                     rowacc, split);
  return hipGetLastError();
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

// one wave per identity row (b, sign, i)
__global__ __launch_bounds__(256) void identity_linear_kernel(const float* __restrict__ W, int n_out, int n_in,
                                                              const float* __restrict__ bias_start,
                                                              const float* __restrict__ lo,
                                                              const float* __restrict__ hi,
                                                              const float* __restrict__ bias_z, int batch,
                                                              float* __restrict__ lam,
                                                              float* __restrict__ rowacc) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int R = 2 * n_out;
  if (row >= (long long)batch * R) return;
  const long long b = row / R;
  const int r = (int)(row - b * R);
  const int i = r < n_out ? r : r - n_out;
  const float sg = r < n_out ? 1.f : -1.f;
  const float* w = W + (long long)i * n_in;
  const float* lb = lo + b * n_in;
  const float* ub = hi + b * n_in;
  float* dst = lam + row * n_in;
  float s = 0.f;
  for (int j = lane; j < n_in; j += 64) {
    float psi = sg * w[j];
    float a, sl, t;
    relax_coeffs(lb[j], ub[j], a, sl, t);
    float o = psi >= 0.f ? psi * a : psi * sl;
    dst[j] = o;
    if (bias_z) s += o * bias_z[j];
    s += fminf(psi, 0.f) * t;
  }
  s = wave_sum(s);
  if (lane == 0) rowacc[row] = (bias_start ? sg * bias_start[i] : 0.f) + s;
}

hipError_t launch_identity_linear(const float* W, int n_out, int n_in, const float* bias_start, const float* lo,
                                  const float* hi, const float* bias_z, int batch, float* lam, float* rowacc,
                                  hipStream_t st) {
  long long rows = (long long)batch * 2 * n_out;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(identity_linear_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, W, n_out, n_in,
                     bias_start, lo, hi, bias_z, batch, lam, rowacc);
  return hipGetLastError();
}

__global__ void identity_fill_kernel(int batch, int n, float* __restrict__ lam) {
  const long long total = (long long)batch * 2 * n * n;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    long long row = e / n;
    int col = (int)(e - row * n);
    int r = (int)(row % (2 * n));
    float v = 0.f;
    if (r < n && col == r) v = 1.f;
    if (r >= n && col == r - n) v = -1.f;
    lam[e] = v;
  }
}

hipError_t launch_identity_fill(int batch, int n, float* lam, hipStream_t st) {
  hipLaunchKernelGGL(identity_fill_kernel, dim3(4096), dim3(256), 0, st, batch, n, lam);
  return hipGetLastError();
}

// one block (256 threads) per row
__global__ __launch_bounds__(256) void relax_kernel(const float* __restrict__ src, int src_broadcast,
                                                    float scale, const float* __restrict__ addend, int rows,
                                                    int rows_per_b, int P, int N, const float* __restrict__ lo,
                                                    const float* __restrict__ hi,
                                                    const float* __restrict__ bias_z,
                                                    const float* __restrict__ alpha, float* __restrict__ psi_out,
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
    if (alpha && l < 0.f && u > 0.f) a = alpha[(long long)row * L + e];
    const float o = v >= 0.f ? v * a : v * sl;
    out[(long long)row * L + e] = o;
    if (psi_out) psi_out[(long long)row * L + e] = v;
    if (bias_z) s += o * bias_z[n];
    s += fminf(v, 0.f) * t;
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) rowacc[row] += s;
}

hipError_t launch_relax(const float* src, int src_broadcast, float scale, const float* addend, int rows,
                        int rows_per_b, int P, int N, const float* lo, const float* hi, const float* bias_z,
                        const float* alpha, float* psi_out, float* out, float* rowacc, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(relax_kernel, dim3(rows), dim3(256), 0, st, src, src_broadcast, scale, addend, rows,
                     rows_per_b, P, N, lo, hi, bias_z, alpha, psi_out, out, rowacc);
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
  sc = block_sum(sc, sh);
  sr = block_sum(sr, sh);
  if (threadIdx.x == 0) {
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
  hipLaunchKernelGGL(concretize_rows_kernel, dim3(rows), dim3(256), 0, st, A, n, rows_per_b, center, radius, eps,
                     lo, hi, bias, lb, ub, rowacc);
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

}  // namespace vb

// fp32 MFMA implicit GEMM for CDNA4 (gfx950): CROWN back-substitution and IBP.
//
// The hot operation of CROWN back-substitution (the A matrices of "Scaling
// Neural Network Verification with Tensor Parallelism and Fully Sharded Data
// Parallelism", Sec. 1 and Sec. 4.1) is Psi = Lambda W for Linear nodes and
// Psi = conv^T(Lambda, W) for Conv nodes, followed by the ReLU relaxation with
// slopes taken from intermediate bounds (Sec. 2.1).  Both are one implicit
// GEMM here: an output position gathers its A row from up to 9 shifted
// positions of a channels-last source (one "tap" each) and the reduction runs
// over (tap, channel); a plain GEMM is the one-tap, one-position case.  IBP's
// W c and |W| r share the same kernel (two accumulator sets, one B tile).
//
// Work decomposition: 256 threads = 4 wavefronts of 64 per workgroup, a
// BM x BN output tile, 32-deep K stages double-buffered in LDS.  Each
// wavefront owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 blocks computed
// with v_mfma_f32_32x32x2f32.  LDS rows are K-contiguous (A as [m][k], B as
// [n][k]) and padded to 36 floats, so a lane fetches four consecutive k of its
// row with one 128-bit LDS read and eight lanes of a read cover 32 distinct
// banks.  The B operand is always stored K-contiguous in HBM ([tap][N][K]):
// the host transposes weights once per call where needed.  When every K
// stage lies inside one tap and rows are 16-byte aligned ("fast" path), the
// global loads are float4 with one bounds decision per row and stage;
// otherwise a scalar path handles ragged K, C_in = 3 and odd alignments.
//
// The epilogue applies the ReLU relaxation (or concretisation, or the IBP
// interval arithmetic) to each output element and reduces each output row to
// one partial sum per N-tile; those partials are summed later in a fixed
// order, so results are bitwise reproducible without float atomics.
#include <hip/hip_runtime.h>

#include <cstring>

#include "vb_internal.h"

namespace vb {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int BK = 32;
constexpr int LDK = BK + 4;  // LDS row stride in floats

__device__ __forceinline__ int fdiv(int x, const FastDiv& f) {
  return f.d == 1 ? x : (int)(__umulhi((unsigned)x, f.mul) >> f.shr);
}

// Gather GEMM: tile index m -> (row, pixel q); rows past the last are padding.
struct GPos {
  int row, q;
  bool valid;
};
__device__ __forceinline__ GPos gdecode(const GemmDesc& d, int m) {
  const int t = m >> d.rb_shift;
  const int rb = fdiv(t, d.div_p);
  GPos g;
  g.q = t - rb * d.div_p.d;
  g.row = (rb << d.rb_shift) + (m & ((1 << d.rb_shift) - 1));
  g.valid = m < d.Mt && g.row < d.div_nrows.d;
  if (!g.valid) g.row = g.q = 0;
  return g;
}

struct Pos {
  long long a_base;
  int row, Y, X;
  bool valid;
};

template <bool DENSE>
__device__ __forceinline__ Pos pos_of(const GemmDesc& d, int m) {
  Pos p;
  if (DENSE) {
    p.valid = m < d.M;
    const int mm = p.valid ? m : 0;
    p.a_base = (long long)mm * d.a_row_stride;
    p.row = mm;
    p.Y = p.X = 0;
  } else {
    const GPos g = gdecode(d, m);
    p.valid = g.valid;
    p.Y = fdiv(g.q, d.div_gw);
    p.X = g.q - p.Y * d.gw;
    p.a_base = (long long)g.row * d.a_row_stride;
    p.row = g.row;
  }
  return p;
}

// Tap table entry j, read with static indices only (dynamic indexing of the
// by-value descriptor would make the compiler copy it to scratch).
struct Tap {
  int dy, dx, w;
};
__device__ __forceinline__ Tap tap_of(const GemmDesc& d, int j) {
  Tap t{d.tap_dy[0], d.tap_dx[0], d.tap_w[0]};
#pragma unroll
  for (int i = 1; i < MAX_TAPS; ++i)
    if (j == i) t = Tap{d.tap_dy[i], d.tap_dx[i], d.tap_w[i]};
  return t;
}

// A offset of (position, reduction index k), or -1 for padding.
template <bool DENSE>
__device__ __forceinline__ long long a_off(const GemmDesc& d, const Pos& p, int k) {
  if (!p.valid || k >= d.K) return -1;
  if (DENSE) return p.a_base + k;
  const int j = (d.ntaps == 1) ? 0 : k / d.cs;
  const int c = k - j * d.cs;
  const Tap t = tap_of(d, j);
  const int yy = p.Y * d.sy + t.dy;
  const int xx = p.X * d.sx + t.dx;
  if (yy < 0 || yy >= d.hs || xx < 0 || xx >= d.ws) return -1;
  return p.a_base + ((long long)yy * d.ws + xx) * d.cs + c;
}

// B offset of (k, n) in the [tap][N][cs] layout, or -1.
__device__ __forceinline__ long long b_off(const GemmDesc& d, int k, int n) {
  if (k >= d.K || n >= d.N) return -1;
  const int j = (d.ntaps == 1) ? 0 : k / d.cs;
  const int c = k - j * d.cs;
  return ((long long)tap_of(d, j).w * d.N + n) * d.cs + c;
}

__device__ __forceinline__ float ld1(const float* base, long long off) {
  const bool ok = off >= 0;
  const float v = base[ok ? off : 0];
  return ok ? v : 0.f;
}

template <int AMODE>
__device__ __forceinline__ void a_val(const GemmDesc& d, long long off, float& c, float& r) {
  if (AMODE == A_PLAIN) {
    c = ld1(d.A, off);
    r = 0.f;
  } else if (AMODE == A_IBP_BOX) {
    const float l = ld1(d.A, off), u = ld1(d.A2, off);
    c = (l + u) * 0.5f;
    r = (u - l) * 0.5f;
  } else {
    c = ld1(d.A, off);
    r = d.A2 ? ld1(d.A2, off) : (off >= 0 ? d.eps : 0.f);
  }
}

// Unconditional global float4 load at a clamped offset, zeroed afterwards when
// the element is padding: keeps every load a plain global load (a conditional
// load lets the compiler route zeros through scratch and a flat load).
__device__ __forceinline__ float4 ld4(const float* base, long long off) {
  const bool ok = off >= 0;
  float4 v = *reinterpret_cast<const float4*>(base + (ok ? off : 0));
  return ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Component-wise select of two register values (no address select).
__device__ __forceinline__ float4 pick4(bool p, const float4& a, const float4& b) {
  return make_float4(p ? a.x : b.x, p ? a.y : b.y, p ? a.z : b.z, p ? a.w : b.w);
}

template <int AMODE>
__device__ __forceinline__ void a_val4(const GemmDesc& d, long long off, float4& c, float4& r) {
  if (AMODE == A_PLAIN) {
    c = ld4(d.A, off);
  } else if (AMODE == A_IBP_BOX) {
    const float4 l = ld4(d.A, off);
    const float4 u = ld4(d.A2, off);
    c = make_float4((l.x + u.x) * 0.5f, (l.y + u.y) * 0.5f, (l.z + u.z) * 0.5f, (l.w + u.w) * 0.5f);
    r = make_float4((u.x - l.x) * 0.5f, (u.y - l.y) * 0.5f, (u.z - l.z) * 0.5f, (u.w - l.w) * 0.5f);
  } else {
    c = ld4(d.A, off);
    if (d.A2) {
      r = ld4(d.A2, off);
    } else {
      const float e = off >= 0 ? d.eps : 0.f;
      r = make_float4(e, e, e, e);
    }
  }
}

}  // namespace

// Epilogue addressing variants (compile-time, so that the common case keeps
// its register budget): plain; footprint windows (rows of identity-start
// neurons kept on a window of the target node); compact per-neuron state
// (alpha, kept Psi and Adam moments on unstable neurons only); footprint
// windows whose taps read two Lambda sources (two branches of a residual
// block that meet at the node being concretised over).
enum { V_PLAIN = 0, V_PATCH = 1, V_COMPACT = 2, V_PATCH2 = 3 };

// One workgroup's output tile `tile0` of the descriptor's tile index space
// (tile0 >= the tile count: nothing to do).
template <int BM, int BN, int WM, int WN, bool DENSE, int AMODE, int EPI, bool FAST, int VAR>
__device__ __forceinline__ void gemm_tile(const GemmDesc& d, const int tile0) {
  constexpr int NTHR = WM * WN * 64;
  constexpr int NA = (AMODE == A_PLAIN) ? 1 : 2;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int NR = (AMODE == A_PLAIN) ? 1 : FM;   // radius accumulators (IBP)
  constexpr int NC = (AMODE == A_PLAIN) ? 1 : FN;
  // per-thread load slots
  constexpr int AV = BM * (BK / 4) / NTHR;                 // float4 of A
  constexpr int BV = (BN * (BK / 4) + NTHR - 1) / NTHR;    // float4 of B
  constexpr int AS = BM * BK / NTHR;                       // scalars of A (slow path)
  constexpr int BS = (BN * BK + NTHR - 1) / NTHR;          // scalars of B (slow path)
  static_assert(FM >= 1 && FN >= 1 && AV >= 1, "tile");
  constexpr bool PATCH = VAR == V_PATCH || VAR == V_PATCH2;
  constexpr bool DUAL = VAR == V_PATCH2;
  static_assert(!DUAL || (FAST && !DENSE && AMODE == A_PLAIN), "two sources: fast gather path only");

  __shared__ __attribute__((aligned(16))) float As[2][NA][BM * LDK];
  __shared__ __attribute__((aligned(16))) float Bs[2][BN * LDK];
  __shared__ float red[WN][BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, half = lane >> 5;

  // Within the run of tiles an XCD gets, the N-tiles of an M-tile (or of a
  // group of M-tiles) are next to each other, so the A rows are fetched into
  // one XCD's L2 once.
  const int mt = (d.Mt + BM - 1) / BM;
  const int nt = (d.N + BN - 1) / BN;
  const int ks_n = ((EPI == E_IBP || EPI == E_ADJOINT) && d.ksplit > 1) ? d.ksplit : 1;
  const int total = mt * nt * ks_n;
  if (tile0 >= total) return;
  const int ks = tile0 / (mt * nt);
  const int tile = tile0 - ks * (mt * nt);
  int tm, tn;
  if (nt >= 4) {
    // wide N: groups of 8 M-tiles sweep the N-tiles together, so their A rows
    // stay in L2 while B moves past them (a plain row-major order re-fetched
    // the A rows once per N-tile)
    constexpr int GM = 8;
    const int grp = tile / (GM * nt);
    const int first = grp * GM;
    const int gm = min(GM, mt - first);
    const int idx = tile - grp * GM * nt;
    tn = idx / gm;
    tm = first + (idx - tn * gm);
  } else {
    tm = tile / nt;
    tn = tile - tm * nt;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  if (d.live_cnt) {
    // selected-neuron rows: skip a tile none of whose rows is live
    bool any = false;
    for (int r = tid; r < BM; r += NTHR) {
      const int m = m0 + r;
      int row = -1;
      if (DENSE) {
        if (m < d.M) row = m;
      } else {
        const GPos g = gdecode(d, m);
        if (g.valid) row = g.row;
      }
      if (row >= 0) {
        const int per = 2 * d.live_u;
        const int b = row / per;
        int u = row - b * per;
        if (u >= d.live_u) u -= d.live_u;
        any = any || u < d.live_cnt[b];
      }
    }
    if (!__syncthreads_or(any)) return;
  }

  // register staging of the next K stage
  float4 ra[NA][FAST ? AV : 1];
  float4 rb[FAST ? BV : 1];
  float sa[NA][FAST ? 1 : AS];
  float sb[FAST ? 1 : BS];
  Pos apos[FAST ? AV : 1];
  if (FAST) {
#pragma unroll
    for (int i = 0; i < AV; ++i) apos[i] = pos_of<DENSE>(d, m0 + (tid + NTHR * i) / (BK / 4));
  }

  // Fast path: the K stages run through the taps in order, 32 channels at a
  // time, so a thread's A and B addresses are worked out once per tap (the
  // gather's bounds test included) and each stage only adds its channel
  // offset.  A dense GEMM is the one-tap case with the whole K as channels.
  long long abase[FAST ? AV : 1], bbase[FAST ? BV : 1];
  int ld_j = 0, ld_c = 0;  // tap and channel offset of the next stage to load
  unsigned tmask = (1u << MAX_TAPS) - 1;  // taps whose stages this workgroup runs
  bool src1 = false;                      // the current tap reads the second source
  auto set_tap = [&](int j) {
    const Tap tp = DENSE ? Tap{0, 0, 0} : tap_of(d, j);
    src1 = DUAL && j >= d.tap_src1;
    const int hs = src1 ? d.hs1 : d.hs, wsrc = src1 ? d.ws1 : d.ws;
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      const int f = tid + NTHR * i;
      const int kq = (f % (BK / 4)) * 4;
      const Pos& p = apos[i];
      long long off = -1;
      if (p.valid) {
        if (DENSE) {
          off = p.a_base + kq;
        } else {
          const int yy = p.Y * d.sy + tp.dy;
          const int xx = p.X * d.sx + tp.dx;
          const long long base = src1 ? (long long)p.row * d.a1_row_stride : p.a_base;
          if (yy >= 0 && yy < hs && xx >= 0 && xx < wsrc) off = base + ((long long)yy * wsrc + xx) * d.cs + kq;
        }
      }
      abase[i] = off;
    }
    const long long bt = (long long)tp.w * d.N;
#pragma unroll
    for (int i = 0; i < BV; ++i) {
      const int f = tid + NTHR * i;
      const int n = f / (BK / 4), kq = (f % (BK / 4)) * 4;
      const bool ok = f < BN * (BK / 4) && n0 + n < d.N;
      bbase[i] = ok ? (bt + n0 + n) * d.cs + kq : -1;
    }
  };

  auto load = [&](int k0) {
    if (FAST) {
      (void)k0;
#pragma unroll
      for (int i = 0; i < AV; ++i) {
        if (DUAL) {
          ra[0][i] = ld4(src1 ? d.A1 : d.A, abase[i] >= 0 ? abase[i] + ld_c : -1);
        } else {
          float4 r4;
          a_val4<AMODE>(d, abase[i] >= 0 ? abase[i] + ld_c : -1, ra[0][i], r4);
          if (NA == 2) ra[NA - 1][i] = r4;
        }
      }
      const float* bsrc = (DUAL && src1) ? d.B1 : d.B;
#pragma unroll
      for (int i = 0; i < BV; ++i) rb[i] = ld4(bsrc, bbase[i] >= 0 ? bbase[i] + ld_c : -1);
      // advance to the next stage: the next 32 channels, or the next tap this
      // tile reads
      ld_c += BK;
      if (!DENSE && ld_c >= d.cs) {
        ld_c = 0;
        const unsigned rest = tmask >> (ld_j + 1);
        ld_j = rest ? ld_j + __ffs(rest) : d.ntaps;
        if (ld_j < d.ntaps) set_tap(ld_j);
      }
    } else {
#pragma unroll
      for (int i = 0; i < AS; ++i) {
        const int e = tid + NTHR * i;
        const Pos p = pos_of<DENSE>(d, m0 + e / BK);
        float c, r;
        a_val<AMODE>(d, a_off<DENSE>(d, p, k0 + (e % BK)), c, r);
        sa[0][i] = c;
        if (NA == 2) sa[NA - 1][i] = r;
      }
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        const int e = tid + NTHR * i;
        sb[i] = ld1(d.B, e < BN * BK ? b_off(d, k0 + (e % BK), n0 + e / BK) : -1);
      }
    }
  };
  auto store = [&](int buf) {
    if (FAST) {
#pragma unroll
      for (int i = 0; i < AV; ++i) {
        const int f = tid + NTHR * i;
        const int row = f / (BK / 4), kq = (f % (BK / 4)) * 4;
        *reinterpret_cast<float4*>(&As[buf][0][row * LDK + kq]) = ra[0][i];
        if (NA == 2) *reinterpret_cast<float4*>(&As[buf][NA - 1][row * LDK + kq]) = ra[NA - 1][i];
      }
#pragma unroll
      for (int i = 0; i < BV; ++i) {
        const int f = tid + NTHR * i;
        if (f < BN * (BK / 4)) {
          const int n = f / (BK / 4), kq = (f % (BK / 4)) * 4;
          *reinterpret_cast<float4*>(&Bs[buf][n * LDK + kq]) = rb[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < AS; ++i) {
        const int e = tid + NTHR * i;
        As[buf][0][(e / BK) * LDK + (e % BK)] = sa[0][i];
        if (NA == 2) As[buf][NA - 1][(e / BK) * LDK + (e % BK)] = sa[NA - 1][i];
      }
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        const int e = tid + NTHR * i;
        if (e < BN * BK) Bs[buf][(e / BK) * LDK + (e % BK)] = sb[i];
      }
    }
  };

  f32x16 acc[FM][FN];
  f32x16 accr[NR][NC];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) accr[i][j][v] = 0.f;

  // K stages of this workgroup (all of them unless IBP splits K)
  const int nk_all = (d.K + BK - 1) / BK;
  const int per_slice = (nk_all + ks_n - 1) / ks_n;
  const int kb = ks * per_slice;
  int nk = min(nk_all - kb, per_slice);
  // Taps that no row of this tile reads inside the source add only zero
  // products: a gather GEMM on the fast path (K not split) runs the stages of
  // the other taps only.  A tap counts for a row if its source cell lies in the
  // source grid (and, for footprint windows, in the source node's image), and
  // the row's own output cell lies in the target image (footprint windows:
  // outside it the epilogue keeps nothing).
  if (FAST && !DENSE && ks_n == 1) {
    __shared__ unsigned tap_mask;
    // taps row m (at position p) reads inside the source
    auto taps_of = [&](const Pos& p, int m) -> unsigned {
      unsigned bits = 0;
      if (!p.valid) return bits;
      int sy0 = 0, sx0 = 0, sy1 = 0, sx1 = 0;
      bool inimg = true;
      if (PATCH) {
        const GPos g = gdecode(d, m);
        const int t1 = fdiv(g.row, d.div_pc);
        const int pz = t1 - fdiv(t1, d.div_pz) * d.div_pz.d;
        const int py = fdiv(pz, d.div_pw), px = pz - py * d.pgw;
        const int ay = py * d.psy + d.poy + p.Y * d.oym + d.oy0;
        const int ax = px * d.psx + d.pox + p.X * d.oxm + d.ox0;
        inimg = ay >= 0 && ay < d.img_h && ax >= 0 && ax < d.img_w;
        sy0 = py * d.ssy + d.soy;
        sx0 = px * d.ssx + d.sox;
        if (DUAL) {
          sy1 = py * d.ssy1 + d.soy1;
          sx1 = px * d.ssx1 + d.sox1;
        }
      }
      if (!inimg) return bits;
      for (int j = 0; j < d.ntaps; ++j) {
        const Tap tp = tap_of(d, j);
        const int yy = p.Y * d.sy + tp.dy, xx = p.X * d.sx + tp.dx;
        const bool s1 = DUAL && j >= d.tap_src1;
        bool ok = yy >= 0 && yy < (s1 ? d.hs1 : d.hs) && xx >= 0 && xx < (s1 ? d.ws1 : d.ws);
        if (s1) {
          if (d.src_h1 > 0)
            ok = ok && sy1 + yy >= 0 && sy1 + yy < d.src_h1 && sx1 + xx >= 0 && sx1 + xx < d.src_w1;
        } else if (PATCH && d.src_h > 0) {
          ok = ok && sy0 + yy >= 0 && sy0 + yy < d.src_h && sx0 + xx >= 0 && sx0 + xx < d.src_w;
        }
        if (ok) bits |= 1u << j;
      }
      return bits;
    };
    unsigned my = 0;
    if (!PATCH || d.pc % 32 == 0) {
      // every row of a 32-row block has the block's output position (and, for
      // footprint rows, its start pixel): one thread per block works it out
      if (tid < BM / 32) my = taps_of(pos_of<DENSE>(d, m0 + 32 * tid), m0 + 32 * tid);
    } else {
#pragma unroll
      for (int i = 0; i < AV; ++i) my |= taps_of(apos[i], m0 + (tid + NTHR * i) / (BK / 4));
    }
    if (tid == 0) tap_mask = 0u;
    __syncthreads();
    if (my) atomicOr(&tap_mask, my);
    __syncthreads();
    tmask = tap_mask;
    nk = __popc(tmask) * (d.cs / BK);
  }
  if (FAST) {
    // first stage of this workgroup's K range
    ld_j = DENSE ? 0 : (kb * BK) / d.cs;
    ld_c = kb * BK - ld_j * d.cs;
    if (!DENSE && ks_n == 1) {
      ld_j = tmask ? __ffs(tmask) - 1 : 0;
      ld_c = 0;
    }
    if (nk > 0) set_tap(ld_j);
  }
  if (nk > 0) {
    load(kb * BK);
    store(0);
  }
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int cur = t & 1;
    if (t + 1 < nk) load((kb + t + 1) * BK);
    // keep the next stage's global loads ahead of this stage's MFMAs and its
    // LDS stores (and their wait for those loads) behind them
    __builtin_amdgcn_sched_barrier(0);
    // MFMA step (q, s): lane half h supplies k = 16h + 4q + s.  On the smaller
    // wave tiles the fragments are double-buffered in registers: the LDS reads
    // of chunk q+1 are issued before the MFMAs of chunk q, so their latency
    // hides behind those MFMAs.  The largest wave tile has no registers to
    // spare for a second set and relies on its 8 MFMAs per read instead.
    constexpr bool DBUF = FM * FN < 8;
    constexpr int NS = DBUF ? 2 : 1;
    float4 fa[NS][FM], fb[NS][FN], fr[NS][NR];
    auto frag = [&](int slot, int q) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[slot][i] = *reinterpret_cast<const float4*>(&As[cur][0][(wm * WTM + i * 32 + l32) * LDK + 16 * half + 4 * q]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[slot][j] = *reinterpret_cast<const float4*>(&Bs[cur][(wn * WTN + j * 32 + l32) * LDK + 16 * half + 4 * q]);
      if (NA == 2) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
          fr[slot][i] = *reinterpret_cast<const float4*>(
              &As[cur][NA - 1][(wm * WTM + i * 32 + l32) * LDK + 16 * half + 4 * q]);
      }
    };
    if (DBUF) frag(0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int sl = DBUF ? (q & 1) : 0;
      if (DBUF && q < 3) frag(sl ^ 1, q + 1);
      if (!DBUF) frag(0, q);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[sl][i][s], fb[sl][j][s], acc[i][j], 0, 0, 0);
        if (NA == 2) {
#pragma unroll
          for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int j = 0; j < NC; ++j)
              accr[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fr[sl][i][s], fabsf(fb[sl][j][s]), accr[i][j], 0, 0, 0);
        }
      }
      if (DBUF && q < 3) {
        // keep the reads of chunk q+1 in front of this chunk's MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, FM + FN + (NA == 2 ? NR : 0), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * FM * FN * NA, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // A concretisation tile none of whose taps reaches any of its rows (a window
  // cell outside the image, say) has only zero products: with nothing added
  // and nothing stored per element, each of its rows' partials is 0.
  if (EPI == E_CONCRETIZE && FAST && !DENSE && ks_n == 1 && nk == 0 && !d.addend && !d.psi_out) {
    if (d.part) {
      for (int r = tid; r < BM; r += NTHR) {
        const GPos gp = gdecode(d, m0 + r);
        if (gp.valid) d.part[((long long)gp.q * d.div_nrows.d + gp.row) * d.part_ld + tn] = 0.f;
      }
    }
    return;
  }
  // The same for a footprint relaxation tile: every product is zero, so every
  // output (and kept Psi) is 0 and so is every row's partial.
  if (EPI == E_RELAX && PATCH && FAST && ks_n == 1 && nk == 0 && !d.addend && !d.alpha) {
    const int HW = d.ho * d.wo;
    const bool v4 = (d.N & 3) == 0;  // (Lambda buffers are 16-byte aligned)
    constexpr int Q = BN / 4;        // float4 per tile row
    for (int e = tid; e < BM * Q; e += NTHR) {
      const int r = e / Q, nn = n0 + 4 * (e - r * Q);
      const GPos gp = gdecode(d, m0 + r);
      if (!gp.valid || nn >= d.N) continue;
      const int Y = fdiv(gp.q, d.div_gw);
      const int X = gp.q - Y * d.gw;
      const long long o =
          ((long long)gp.row * HW + (long long)(Y * d.oym + d.oy0) * d.wo + (X * d.oxm + d.ox0)) * d.N + nn;
      if (v4) {
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(d.out + o) = z;
        if (d.psi_out) *reinterpret_cast<float4*>(d.psi_out + o) = z;
      } else {
        for (int c = 0; c < 4 && nn + c < d.N; ++c) {
          d.out[o + c] = 0.f;
          if (d.psi_out) d.psi_out[o + c] = 0.f;
        }
      }
    }
    if (d.part) {
      for (int r = tid; r < BM; r += NTHR) {
        const GPos gp = gdecode(d, m0 + r);
        if (gp.valid) d.part[((long long)gp.q * d.div_nrows.d + gp.row) * d.part_ld + tn] = 0.f;
      }
    }
    return;
  }

  // ---- epilogue.  (Every multiply-add below is an explicit fmaf, so that each
  // instantiation rounds alike whatever the compiler's contraction choices.)
  // Register v of lane l of a 32x32 fp32 MFMA result holds
  // row 8*(v/4) + 4*(l/32) + v%4 and column l%32 of the block.  The elements
  // are handled 8 rows at a time: indices first (clamped in range), then every
  // load of the group (unconditional, so they can all be in flight together),
  // then the arithmetic with predicated stores.
  constexpr bool ROWSUM = (EPI != E_IBP && EPI != E_ADJOINT);
  // rows per group (fewer where registers are short)
  constexpr int G = (FM * FN >= 2 || VAR == V_COMPACT) ? 4 : 8;
  // The 32 rows of a block i of a gather tile lie in one block of 2^rb_shift
  // >= 32 rows of the same output position: the position (and its division
  // work) is decoded once per block, and each element only adds its row
  // offset.  Footprint rows (b, sign, start pixel, channel) share their start
  // pixel across a 32-row block when the start node's channel count is a
  // multiple of 32, so their window-cell-to-pixel decode is also once per
  // block; otherwise it is per row.
  constexpr bool one_pos = !DENSE && !PATCH;
  const bool blk = one_pos || (PATCH && d.pc % 32 == 0);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    int row0 = 0, r0 = 0, b0 = 0;
    long long obase = 0, bbase = 0;  // element offsets of (r0, position) in the output and in coef
    bool blk_ok = false, pin_blk = true;
    const int HWN = d.ho * d.wo * d.N;  // elements per row (the host keeps 32 * HWN < 2^31)
    if (blk) {
      const GPos gp = gdecode(d, m0 + wm * WTM + i * 32);
      blk_ok = m0 + wm * WTM + i * 32 < d.Mt;
      row0 = gp.row;
      const int Y = fdiv(gp.q, d.div_gw);
      const int X = gp.q - Y * d.gw;
      const int cy = Y * d.oym + d.oy0, cx = X * d.oxm + d.ox0;
      const long long sp0 = (long long)cy * d.wo + cx;
      // padding rows address row r0 (a valid row) and are never stored
      r0 = min(row0, d.div_nrows.d - 1);
      b0 = fdiv(r0, d.div_rows);
      obase = ((long long)r0 * d.ho * d.wo + sp0) * d.N;
      if (PATCH) {
        // window cell -> pixel of the target node for the block's start pixel
        const int t1 = fdiv(r0, d.div_pc);
        const int pz = t1 - fdiv(t1, d.div_pz) * d.div_pz.d;
        const int py = fdiv(pz, d.div_pw), px = pz - py * d.pgw;
        const int ay = py * d.psy + d.poy + cy, ax = px * d.psx + d.pox + cx;
        pin_blk = ay >= 0 && ay < d.img_h && ax >= 0 && ax < d.img_w;
        bbase = ((long long)b0 * d.img_h * d.img_w + (pin_blk ? (long long)ay * d.img_w + ax : 0)) * d.N;
      } else {
        bbase = ((long long)b0 * d.ho * d.wo + sp0) * d.N;
      }
    }
    // Per-neuron data of an element (relaxation coefficients, domain centre and
    // radius) depends on its batch element, position and column only.  The 32
    // rows of a block share their position (and, for footprint rows, their input),
    // and with at least 32 rows per batch element they span at most two batch
    // elements: each column's data is then read once per block for those two and
    // selected per row, instead of once per element.
    constexpr bool NEEDS_B = EPI == E_RELAX || EPI == E_ADJOINT || EPI == E_CONCRETIZE;
    const bool hoist = NEEDS_B && (DENSE || blk) && (PATCH || d.rows_per_b >= 32);
    long long hb0 = 0, hb1 = 0;  // data offsets (column 0) of the block's first and second batch element
    bool two = false;
    int hbA = 0;                 // dense: batch element of the block's first row
    if (NEEDS_B && hoist) {
      if (DENSE) {
        const int mf = m0 + wm * WTM + i * 32;
        hbA = fdiv(min(mf, d.M - 1), d.div_rows);
        two = fdiv(min(mf + 31, d.M - 1), d.div_rows) != hbA;
        hb0 = (long long)hbA * d.N;
        hb1 = hb0 + d.N;
      } else {
        hb0 = bbase;
        hb1 = bbase + HWN;
        two = !PATCH && fdiv(min(row0 + 31, d.div_nrows.d - 1), d.div_rows) != b0;
      }
    }
    float4 hc0[(EPI == E_RELAX || EPI == E_ADJOINT) ? FN : 1], hc1[(EPI == E_RELAX || EPI == E_ADJOINT) ? FN : 1];
    float hcen0[EPI == E_CONCRETIZE ? FN : 1], hcen1[EPI == E_CONCRETIZE ? FN : 1];
    float hrad0[EPI == E_CONCRETIZE ? FN : 1], hrad1[EPI == E_CONCRETIZE ? FN : 1];
    if (NEEDS_B && hoist) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WTN + j * 32 + l32;
        const int nn = n < d.N ? n : 0;
        if (EPI == E_RELAX || EPI == E_ADJOINT) {
          hc0[j] = d.coef[hb0 + nn];
          hc1[j] = d.coef[two ? hb1 + nn : hb0 + nn];
        } else if (EPI == E_CONCRETIZE) {
          hcen0[j] = d.center[hb0 + nn];
          hcen1[j] = d.center[two ? hb1 + nn : hb0 + nn];
          hrad0[j] = d.radius ? d.radius[hb0 + nn] : d.eps;
          hrad1[j] = d.radius ? d.radius[two ? hb1 + nn : hb0 + nn] : d.eps;
        }
      }
    }
#pragma unroll
    for (int v0 = 0; v0 < 16; v0 += G) {
      long long opos[G], bpos[G];
      int rbase[G];  // compact per-neuron state: first entry of the element's row
      bool mok[G], pin[G], sel[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int v = v0 + g;
        const int m = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        pin[g] = true;
        if (blk) {
          // offsets from (r0, position): 32-bit arithmetic per element
          const int row = row0 + 8 * (v >> 2) + 4 * half + (v & 3);
          mok[g] = blk_ok && row < d.div_nrows.d;
          const int rr = mok[g] ? row : r0;
          rbase[g] = rr * d.acols;
          opos[g] = (rr - r0) * HWN;
          // (footprint rows of a block share their input and start pixel)
          bpos[g] = PATCH ? 0 : (fdiv(rr, d.div_rows) - b0) * HWN;
          sel[g] = bpos[g] != 0;
          pin[g] = pin_blk;
        } else if (DENSE) {
          mok[g] = m < d.M;
          const int mm = mok[g] ? m : 0;
          opos[g] = mm;
          rbase[g] = mm * d.acols;
          bpos[g] = fdiv(mm, d.div_rows);
          sel[g] = bpos[g] != hbA;
        } else {
          sel[g] = false;
          const GPos gp = gdecode(d, m);
          mok[g] = gp.valid;
          rbase[g] = gp.row * d.acols;
          const int Y = fdiv(gp.q, d.div_gw);
          const int X = gp.q - Y * d.gw;
          const int cy = Y * d.oym + d.oy0, cx = X * d.oxm + d.ox0;
          const long long sp = (long long)cy * d.wo + cx;
          opos[g] = (long long)gp.row * d.ho * d.wo + sp;
          const long long b = fdiv(gp.row, d.div_rows);
          if (PATCH) {
            // window cell -> pixel of the target node for the row's own position
            const int t1 = fdiv(gp.row, d.div_pc);
            const int pz = t1 - fdiv(t1, d.div_pz) * d.div_pz.d;
            const int py = fdiv(pz, d.div_pw), px = pz - py * d.pgw;
            const int ay = py * d.psy + d.poy + cy, ax = px * d.psx + d.pox + cx;
            pin[g] = ay >= 0 && ay < d.img_h && ax >= 0 && ax < d.img_w;
            bpos[g] = b * d.img_h * d.img_w + (pin[g] ? (long long)ay * d.img_w + ax : 0);
          } else {
            bpos[g] = b * d.ho * d.wo + sp;
          }
        }
      }
      float rowsum[G];
#pragma unroll
      for (int g = 0; g < G; ++g) rowsum[g] = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WTN + j * 32 + l32;
        const bool nok = n < d.N;
        const int nn = nok ? n : 0;
        const int nb = d.bias_c ? nn % d.bias_c : nn;
        const float bias = d.bias ? d.bias[nb] : 0.f;
        long long oi[G], bi[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (blk) {
            oi[g] = obase + (unsigned)((int)opos[g] + nn);
            bi[g] = bbase + (unsigned)((int)bpos[g] + nn);
          } else {
            oi[g] = opos[g] * d.N + nn;
            bi[g] = bpos[g] * d.N + nn;
          }
        }
        // per-neuron state (alpha, kept Psi, Adam moments): at oi, or in the
        // compact layout at the neuron's column of the element's row (the column
        // comes with the relaxation coefficients; the host keeps rows * acols < 2^31)
        auto state_at = [&](int g, int col) -> long long {
          return VAR == V_COMPACT ? (long long)(unsigned)(rbase[g] + (col > 0 ? col : 0)) : oi[g];
        };
        float val[G];
#pragma unroll
        for (int g = 0; g < G; ++g) val[g] = acc[i][j][v0 + g];
        if (EPI == E_IBP) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (!(mok[g] && nok)) continue;
            const float rr = accr[NR == 1 ? 0 : i][NC == 1 ? 0 : j][v0 + g];
            if (ks_n > 1) {
              const long long so = (long long)ks * d.M * d.N;
              d.out[so + oi[g]] = val[g];
              d.out2[so + oi[g]] = rr;
            } else {
              const float cc = val[g] + bias;
              const float l = cc - rr, u = cc + rr;
              d.out[oi[g]] = l;
              d.out2[oi[g]] = u;
              if (d.relu_lo) {
                d.relu_lo[oi[g]] = fmaxf(l, 0.f);
                d.relu_hi[oi[g]] = fmaxf(u, 0.f);
              }
            }
          }
          continue;
        }
        if (EPI == E_ADJOINT && ks_n > 1) {
          // split K: raw products of this slice (summed by launch_adjoint_finish)
          const long long so = (long long)ks * d.M * d.N;
#pragma unroll
          for (int g = 0; g < G; ++g)
            if (mok[g] && nok) d.out[so + oi[g]] = val[g];
          continue;
        }
        if (d.addend) {
          float ad[G];
#pragma unroll
          for (int g = 0; g < G; ++g) ad[g] = d.addend[oi[g]];
#pragma unroll
          for (int g = 0; g < G; ++g) val[g] += ad[g];
        }
        if (EPI == E_STORE) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (mok[g] && nok) {
              d.out[oi[g]] = val[g];
              rowsum[g] = fmaf(val[g], bias, rowsum[g]);
            }
          }
        } else if (EPI == E_RELAX) {
          float4 cf[G];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            cf[g] = hoist ? pick4(sel[g], hc1[j], hc0[j]) : d.coef[bi[g]];
            if (!pin[g]) cf[g] = make_float4(0.f, 0.f, 0.f, __int_as_float(-1));  // outside the node: no neuron
          }
          // slope of the lower relaxation: the optimised alpha on unstable
          // neurons (coefficient column >= 0) when one is given, else the adaptive choice
          float al[G];
#pragma unroll
          for (int g = 0; g < G; ++g) al[g] = cf[g].x;
          if (d.alpha) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
              // (compact state: stable neurons have no entry and load nothing)
              const int col = __float_as_int(cf[g].w);
              if (VAR == V_COMPACT) {
                if (col >= 0) al[g] = d.alpha[state_at(g, col)];
              } else {
                const float t = d.alpha[state_at(g, col)];
                al[g] = col >= 0 ? t : al[g];
              }
            }
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float a = al[g];
            const float o = (val[g] >= 0.f) ? val[g] * a : val[g] * cf[g].y;
            if (mok[g] && nok) {
              d.out[oi[g]] = o;
              const int col = __float_as_int(cf[g].w);
              if (d.psi_out && (VAR != V_COMPACT || col >= 0)) d.psi_out[state_at(g, col)] = val[g];
              rowsum[g] = fmaf(fminf(val[g], 0.f), cf[g].z, fmaf(o, bias, rowsum[g]));
            }
          }
        } else if (EPI == E_ADJOINT) {
          // the accumulator is the adjoint over z: add z's bias
          // (a compact layout without any unstable neuron has no state arrays at all)
          const bool have = d.alpha_rw != nullptr;
          float4 cf[G];
          float psi[G], aold[G], am[G], av[G];
          long long ai[G];
#pragma unroll
          for (int g = 0; g < G; ++g) cf[g] = hoist ? pick4(sel[g], hc1[j], hc0[j]) : d.coef[bi[g]];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            ai[g] = state_at(g, __float_as_int(cf[g].w));
            // (compact state: only unstable neurons have an entry to load)
            const bool ld = have && (VAR != V_COMPACT || __float_as_int(cf[g].w) >= 0);
            psi[g] = ld ? d.psi_in[ai[g]] : 0.f;
            aold[g] = ld ? d.alpha_rw[ai[g]] : 0.f;
            am[g] = av[g] = 0.f;
            if (d.do_update && ld) {
              am[g] = d.adam_m[ai[g]];
              av[g] = d.adam_v[ai[g]];
            }
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float gz = val[g] + bias;
            const bool unstable = __float_as_int(cf[g].w) >= 0 && have;
            // stable neurons: a = s (0 inactive, 1 active); unstable: the Psi >= 0 branch takes alpha
            const float o = !unstable ? gz * cf[g].y : (psi[g] >= 0.f ? gz * aold[g] : fmaf(gz, cf[g].y, cf[g].z));
            if (mok[g] && nok) {
              d.out[oi[g]] = o;
              if (d.gz_out) d.gz_out[oi[g]] = gz;
              if (unstable && d.do_update) {
                const float grad = gz * fmaxf(psi[g], 0.f);
                const float mm = fmaf(d.beta1, am[g], (1.f - d.beta1) * grad);
                const float vv = fmaf(d.beta2, av[g], ((1.f - d.beta2) * grad) * grad);
                d.adam_m[ai[g]] = mm;
                d.adam_v[ai[g]] = vv;
                const float step = d.lr * (mm * d.bc1) / (sqrtf(vv * d.bc2) + d.adam_eps);
                d.alpha_rw[ai[g]] = fminf(fmaxf(aold[g] + step, 0.f), 1.f);
              }
            }
          }
        } else {  // E_CONCRETIZE: centre and radius of the domain box
          float c[G], r[G];
          if (hoist) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
              c[g] = sel[g] ? hcen1[j] : hcen0[j];
              r[g] = sel[g] ? hrad1[j] : hrad0[j];
            }
          } else {
#pragma unroll
            for (int g = 0; g < G; ++g) c[g] = d.center[bi[g]];
            if (d.radius) {
#pragma unroll
              for (int g = 0; g < G; ++g) r[g] = d.radius[bi[g]];
            } else {
#pragma unroll
              for (int g = 0; g < G; ++g) r[g] = d.eps;  // L-infinity ball of one radius
            }
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (!pin[g]) {  // a window cell outside the domain node: no input there
              c[g] = 0.f;
              r[g] = 0.f;
            }
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (mok[g] && nok) {
              if (d.psi_out) d.psi_out[oi[g]] = val[g];
              rowsum[g] = fmaf(-fabsf(val[g]), r[g], fmaf(val[g], c[g], rowsum[g]));
            }
          }
        }
      }
      if (ROWSUM) {
        // Sum each of the G row values over the 32 lanes (columns) of the
        // half-wave, halving the values held per lane at every exchange: at
        // distance 16 a lane keeps half of its rows and adds its partner's
        // copies of them, and so on, G/2 + G/4 + ... + 1 exchanges in all
        // (plus the rest of the butterfly) instead of 5 per row.  A lane then
        // holds the total of row `hr`.
        constexpr int LG = (G == 8) ? 3 : 2;
        float rs[G];
#pragma unroll
        for (int g = 0; g < G; ++g) rs[g] = rowsum[g];
        int hr = 0;
#pragma unroll
        for (int st = 0; st < 5; ++st) {
          const int o = 16 >> st;
          if (st < LG) {
            const int w = G >> (st + 1);  // values kept after this exchange
            const bool up = (l32 & o) != 0;
#pragma unroll
            for (int k = 0; k < w; ++k) {
              const float send = up ? rs[k] : rs[k + w];
              const float keep = up ? rs[k + w] : rs[k];
              rs[k] = keep + __shfl_xor(send, o, 32);
            }
            hr += up ? w : 0;
          } else {
            rs[0] += __shfl_xor(rs[0], o, 32);
          }
        }
        // lanes that agree on bits 4..(5-LG) of l32 hold the same total
        if ((l32 & ((32 >> LG) - 1)) == 0) {
          const int v = v0 + hr;
          red[wn][wm * WTM + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3)] = rs[0];
        }
      }
    }
  }
  if (ROWSUM) {
    __syncthreads();
    if (d.part) {
      for (int r = tid; r < BM; r += NTHR) {
        const int m = m0 + r;
        long long pm = m;
        bool ok = m < d.M;
        if (!DENSE) {
          const GPos gp = gdecode(d, m);
          ok = gp.valid;
          pm = (long long)gp.q * d.div_nrows.d + gp.row;  // position-major partial row
        }
        if (ok) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < WN; ++w) s += red[w][r];
          d.part[pm * d.part_ld + tn] = s;
        }
      }
    }
  }
}

// Tile count of a descriptor's tile index space for a BM x BN tile.
template <int BM, int BN, int EPI>
__host__ __device__ __forceinline__ int tile_count(const GemmDesc& d) {
  const int ks_n = ((EPI == E_IBP || EPI == E_ADJOINT) && d.ksplit > 1) ? d.ksplit : 1;
  return ((d.Mt + BM - 1) / BM) * ((d.N + BN - 1) / BN) * ks_n;
}

// XCD-aware tile order: workgroups go round-robin over the 8 XCDs, so each
// XCD gets a contiguous run of tiles.
template <int BM, int BN, int WM, int WN, bool DENSE, int AMODE, int EPI, bool FAST, int VAR = V_PLAIN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(const GemmDesc d) {
  const int per_xcd = (tile_count<BM, BN, EPI>(d) + 7) / 8;
  gemm_tile<BM, BN, WM, WN, DENSE, AMODE, EPI, FAST, VAR>(d, (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3));
}

// Several GEMMs of one shape family in one grid (the output-parity classes of a
// strided transposed convolution): each XCD takes a contiguous run of every
// class's tiles, the classes one after the other in the order given (longest
// reduction first, so that the short tiles fill the end of the grid).
template <int BM, int BN, int WM, int WN, bool DENSE, int AMODE, int EPI, bool FAST, int VAR = V_PLAIN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_multi_kernel(const GemmMulti mm) {
  const int slot = blockIdx.x >> 3;
  int c = 0;
#pragma unroll
  for (int i = 1; i < MAX_GEMM_MULTI; ++i)
    if (i < mm.n && slot >= mm.first[i]) c = i;
  const int per_xcd = mm.first[c + 1] - mm.first[c];
  gemm_tile<BM, BN, WM, WN, DENSE, AMODE, EPI, FAST, VAR>(mm.d[c], (blockIdx.x & 7) * per_xcd + (slot - mm.first[c]));
}

namespace {

template <int BM, int BN, int WM, int WN, bool DENSE, bool FAST>
hipError_t launch_tile(const GemmDesc& d, hipStream_t st) {
  const int mt = (d.Mt + BM - 1) / BM;
  const int nt = (d.N + BN - 1) / BN;
  const int ks = ((d.epi == E_IBP || d.epi == E_ADJOINT) && d.ksplit > 1) ? d.ksplit : 1;
  const dim3 g(((mt * nt * ks + 7) / 8) * 8), b(WM * WN * 64);
  switch (d.epi) {
    case E_STORE:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_STORE, FAST>), g, b, 0, st, d);
      break;
    case E_RELAX:
      if (!DENSE && d.patch)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_RELAX, FAST, DENSE ? V_PLAIN : V_PATCH>), g, b, 0,
                           st, d);
      else if (d.aidx)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_RELAX, FAST, V_COMPACT>), g, b, 0, st, d);
      else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_RELAX, FAST>), g, b, 0, st, d);
      break;
    case E_CONCRETIZE:
      if (!DENSE && FAST && d.patch && d.A1)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, false, A_PLAIN, E_CONCRETIZE, true, V_PATCH2>), g, b, 0, st, d);
      else if (!DENSE && d.patch)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_CONCRETIZE, FAST, DENSE ? V_PLAIN : V_PATCH>), g, b,
                           0, st, d);
      else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_CONCRETIZE, FAST>), g, b, 0, st, d);
      break;
    case E_ADJOINT:
      if (d.aidx)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_ADJOINT, FAST, V_COMPACT>), g, b, 0, st, d);
      else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_PLAIN, E_ADJOINT, FAST>), g, b, 0, st, d);
      break;
    case E_IBP:
      if (d.amode == A_IBP_BOX)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_IBP_BOX, E_IBP, FAST>), g, b, 0, st, d);
      else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, DENSE, A_IBP_BALL, E_IBP, FAST>), g, b, 0, st, d);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_shape(const GemmDesc& d, bool dense, bool fast, hipStream_t st) {
  if (dense) return fast ? launch_tile<BM, BN, WM, WN, true, true>(d, st) : launch_tile<BM, BN, WM, WN, true, false>(d, st);
  return fast ? launch_tile<BM, BN, WM, WN, false, true>(d, st) : launch_tile<BM, BN, WM, WN, false, false>(d, st);
}

// 256 x 256 tiles on 8 wavefronts (128 x 64 each) for the large convolution
// GEMMs with the fast path, when the grid still has at least two workgroups per CU
// (dense GEMMs ran faster on two 128 x 128 workgroups per CU).
bool use_big(const GemmDesc& d, bool fast) {
  // (the 256 x 256 variants exist for the store, relaxation and concretisation
  // epilogues only)
  if (d.epi != E_STORE && d.epi != E_RELAX && d.epi != E_CONCRETIZE) return false;
  if (!fast || d.N < 256 || gemm_is_dense(d) || d.patch || d.aidx) return false;
  const long long tiles = (long long)((d.Mt + 255) / 256) * ((d.N + 255) / 256);
  return tiles >= 512;
}

int tile_n(const GemmDesc& d, bool fast) {
  if (use_big(d, fast)) return 256;
  return d.N > 64 ? 128 : (d.N > 32 ? 64 : 32);
}

bool is_fast(const GemmDesc& d);

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

namespace {
// fast path: every 32-deep K stage inside one tap, float4-aligned rows
bool is_fast(const GemmDesc& d) {
  return d.K > 0 && d.cs % BK == 0 && d.a_row_stride % 4 == 0 && aligned16(d.A) &&
         (d.A2 == nullptr || aligned16(d.A2)) && aligned16(d.B) &&
         (d.A1 == nullptr || (aligned16(d.A1) && aligned16(d.B1) && d.a1_row_stride % 4 == 0));
}
}  // namespace

namespace {
// Launch-time fields of a descriptor: division constants and the tile index space.
bool finalize(GemmDesc& d) {
  d.div_p = make_fastdiv(d.gh * d.gw);
  d.div_gw = make_fastdiv(d.gw);
  d.div_rows = make_fastdiv(d.rows_per_b);
  d.div_nrows = make_fastdiv(d.M / (d.gh * d.gw));
  if (d.patch) {
    d.div_pc = make_fastdiv(d.pc);
    d.div_pz = make_fastdiv(d.pgh * d.pgw);
    d.div_pw = make_fastdiv(d.pgw);
  }
  d.Mt = d.M;
  d.rb_shift = 0;
  if (!gemm_is_dense(d)) {
    // blocks of 64 rows, or 32 where padding the rows to a whole block of 64
    // would waste more than an eighth of the tiles (the epilogue decodes one
    // output position per 32 rows)
    const long long rows = d.M / (d.gh * d.gw), P = (long long)d.gh * d.gw;
    int sh = 6;
    if (d.patch && rows % 128 == 0) {
      // footprint rows: a 128-row tile then holds one window cell of 128
      // consecutive rows (one start pixel when it has >= 128 channels), so all
      // its rows read the same taps and the tap mask skips exactly what none of
      // them reads
      sh = 7;
    } else if ((((rows + 63) >> 6 << 6) - rows) * 8 > rows) {
      sh = 5;
    }
    const long long mt = ((rows + (1LL << sh) - 1) >> sh << sh) * P;
    if (mt > INT32_MAX - 256) return false;
    // the epilogue's per-block element offsets are 32-bit
    if (32LL * d.ho * d.wo * d.N >= (1LL << 31)) return false;
    d.rb_shift = sh;
    d.Mt = (int)mt;
  }
  return true;
}
}  // namespace

int gemm_ntiles(const GemmDesc& desc) {
  GemmDesc d = desc;
  finalize(d);  // the N-tile width can depend on the tile count
  const int bn = tile_n(d, is_fast(d));
  return (d.N + bn - 1) / bn;
}

namespace {
template <int BM, int BN, int WM, int WN>
hipError_t launch_multi_shape(const GemmMulti& mm, hipStream_t st) {
  const GemmDesc& d = mm.d[0];
  const dim3 g(8 * mm.first[mm.n]), b(WM * WN * 64);
  switch (d.epi) {
    case E_STORE:
      hipLaunchKernelGGL((gemm_multi_kernel<BM, BN, WM, WN, false, A_PLAIN, E_STORE, true>), g, b, 0, st, mm);
      break;
    case E_RELAX:
      if (d.aidx)
        hipLaunchKernelGGL((gemm_multi_kernel<BM, BN, WM, WN, false, A_PLAIN, E_RELAX, true, V_COMPACT>), g, b, 0, st, mm);
      else
        hipLaunchKernelGGL((gemm_multi_kernel<BM, BN, WM, WN, false, A_PLAIN, E_RELAX, true>), g, b, 0, st, mm);
      break;
    case E_CONCRETIZE:
      hipLaunchKernelGGL((gemm_multi_kernel<BM, BN, WM, WN, false, A_PLAIN, E_CONCRETIZE, true>), g, b, 0, st, mm);
      break;
    default:
      return hipErrorNotSupported;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_multi(const GemmDesc* ds, int n, hipStream_t st) {
  if (n < 1 || n > MAX_GEMM_MULTI) return hipErrorInvalidValue;
  GemmMulti mm;
  std::memset(&mm, 0, sizeof mm);
  int bn = 0;
  for (int c = 0; c < n; ++c) {
    GemmDesc d = ds[c];
    if (d.M <= 0 || d.N <= 0) return hipErrorNotSupported;
    if (!finalize(d)) return hipErrorInvalidValue;
    // plain gather GEMMs on the fast path with one epilogue variant
    if (gemm_is_dense(d) || !is_fast(d) || d.patch || d.A1 || d.amode != A_PLAIN) return hipErrorNotSupported;
    if (d.epi != E_STORE && d.epi != E_RELAX && d.epi != E_CONCRETIZE) return hipErrorNotSupported;
    const int t = tile_n(d, true);
    if (t == 256 || (c > 0 && (t != bn || d.epi != mm.d[0].epi || (d.aidx != nullptr) != (mm.d[0].aidx != nullptr))))
      return hipErrorNotSupported;
    bn = t;
    // insertion by reduction length, longest first (ties keep their order)
    int at = c;
    while (at > 0 && mm.d[at - 1].K < d.K) {
      mm.d[at] = mm.d[at - 1];
      --at;
    }
    mm.d[at] = d;
  }
  mm.n = n;
  for (int c = 0; c < n; ++c) {
    const GemmDesc& d = mm.d[c];
    const long long tiles = (long long)((d.Mt + 127) / 128) * ((d.N + bn - 1) / bn);
    mm.first[c + 1] = mm.first[c] + (int)((tiles + 7) / 8);
  }
  if (bn == 128) return launch_multi_shape<128, 128, 4, 2>(mm, st);
  if (bn == 64) return launch_multi_shape<128, 64, 4, 2>(mm, st);
  return launch_multi_shape<128, 32, 4, 1>(mm, st);
}

hipError_t launch_gemm(const GemmDesc& desc, hipStream_t st) {
  if (desc.M <= 0 || desc.N <= 0) return hipSuccess;
  GemmDesc d = desc;
  if (!finalize(d)) return hipErrorInvalidValue;
  const bool dense = gemm_is_dense(d);
  const bool fast = is_fast(d);
  // a second A source exists only as a fast-path footprint concretisation
  if (d.A1 && (!fast || dense || !d.patch || d.epi != E_CONCRETIZE || d.tap_src1 < 0 || d.tap_src1 > d.ntaps))
    return hipErrorInvalidValue;
  const int bn = tile_n(d, fast);
  if (bn == 256) {
    // gather GEMMs with the store, relaxation or concretisation epilogue only
    // (checked in use_big); IBP and the adjoint never take this tile
    const int mt = (d.Mt + 255) / 256, nt = (d.N + 255) / 256;
    const dim3 g(((mt * nt + 7) / 8) * 8), b(512);
    switch (d.epi) {
      case E_STORE: hipLaunchKernelGGL((gemm_kernel<256, 256, 2, 4, false, A_PLAIN, E_STORE, true>), g, b, 0, st, d); break;
      case E_RELAX: hipLaunchKernelGGL((gemm_kernel<256, 256, 2, 4, false, A_PLAIN, E_RELAX, true>), g, b, 0, st, d); break;
      case E_CONCRETIZE:
        hipLaunchKernelGGL((gemm_kernel<256, 256, 2, 4, false, A_PLAIN, E_CONCRETIZE, true>), g, b, 0, st, d);
        break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (bn == 128) return launch_shape<128, 128, 4, 2>(d, dense, fast, st);
  if (bn == 64) return launch_shape<128, 64, 4, 2>(d, dense, fast, st);
  return launch_shape<128, 32, 4, 1>(d, dense, fast, st);
}

}  // namespace vb

// C ABI entry points and the host-side planner of the bound propagation library.
//
// The planner validates the graph, sizes the caller's workspace, and walks
// the graph: forward for IBP, backward for CROWN back-substitution ("Scaling
// Neural Network Verification with Tensor Parallelism and Fully Sharded Data
// Parallelism", Sec. 1: the A matrices; Sec. 2.1: relaxation slopes from
// intermediate bounds; Sec. 2.2: convolutions).  For every Linear / Conv node
// on the backward path it chooses the GEMM epilogue: relax into the ReLU below
// (when this node is that ReLU's last pending consumer), concretise at the
// domain node, or store the product for a later accumulation.  Lambda buffers
// come from a small reference-counted pool inside the workspace; when the
// workspace cannot hold the whole batch, the batch is processed in chunks.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "vb.h"
#include "vb_internal.h"

using namespace vb;

namespace {

thread_local std::string g_err;

vb_status fail(vb_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define HIPCHK(expr)                                                                    \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(VB_EDEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr int NPOOL = 4;
constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct NodeInfo {
  int op, in0, in1;
  int c, h, w;
  long long size;
  int kh, kw, stride, pad;
  const float* W;
  const float* b;
  const float* Wp;        // packed copy of a LINEAR node's W (vb_pack_linear) or NULL
  std::vector<int> cons;  // consumers (direct)
};

struct Graph {
  std::vector<NodeInfo> n;
  int L = 0;  // last node
};

vb_status parse_graph(const vb_graph* g, Graph& G) {
  if (!g || !g->nodes || g->n_nodes < 2) return fail(VB_EINVAL, "graph is NULL or has fewer than 2 nodes");
  const int N = g->n_nodes;
  G.n.resize(N);
  for (int k = 0; k < N; ++k) {
    const vb_node& s = g->nodes[k];
    NodeInfo& d = G.n[k];
    d.op = s.op;
    d.in0 = s.in0;
    d.in1 = s.in1;
    d.c = s.c;
    d.h = s.h;
    d.w = s.w;
    d.kh = s.kh;
    d.kw = s.kw;
    d.stride = s.stride;
    d.pad = s.pad;
    d.W = s.weight;
    d.b = s.bias;
    d.Wp = s.weight_packed;
    if (d.Wp && (s.op != VB_LINEAR || ((uintptr_t)d.Wp & 15) != 0))
      return fail(VB_EINVAL, "node %d: weight_packed is for LINEAR nodes, 16-byte aligned", k);
    if (d.c <= 0 || d.h <= 0 || d.w <= 0) return fail(VB_ESHAPE, "node %d: non-positive shape", k);
    d.size = (long long)d.c * d.h * d.w;
    if (d.size >= (1LL << 31)) return fail(VB_ESHAPE, "node %d: size too large", k);
    if (k == 0) {
      if (d.op != VB_INPUT) return fail(VB_ESHAPE, "node 0 must be VB_INPUT");
      continue;
    }
    if (d.op < VB_INPUT || d.op > VB_FLATTEN) return fail(VB_EINVAL, "node %d: unknown op %d", k, d.op);
    if (d.op == VB_INPUT) return fail(VB_ESHAPE, "node %d: only node 0 may be VB_INPUT", k);
    if (d.in0 < 0 || d.in0 >= k) return fail(VB_ESHAPE, "node %d: in0 %d is not an earlier node", k, d.in0);
    if (d.op == VB_ADD) {
      if (d.in1 < 0 || d.in1 >= k) return fail(VB_ESHAPE, "node %d: in1 %d is not an earlier node", k, d.in1);
    } else if (d.in1 != -1) {
      return fail(VB_ESHAPE, "node %d: in1 must be -1 for this op", k);
    }
    const NodeInfo& p = G.n[d.in0];
    switch (d.op) {
      case VB_LINEAR:
        if (!d.W) return fail(VB_EINVAL, "node %d: linear weight is NULL", k);
        if (p.h != 1 || p.w != 1) return fail(VB_ESHAPE, "node %d: linear input must be flat", k);
        if (d.h != 1 || d.w != 1) return fail(VB_ESHAPE, "node %d: linear output must be flat", k);
        break;
      case VB_CONV2D: {
        if (!d.W) return fail(VB_EINVAL, "node %d: conv weight is NULL", k);
        if (d.kh <= 0 || d.kw <= 0 || d.kh * d.kw > MAX_TAPS || d.stride <= 0 || d.pad < 0)
          return fail(VB_EUNSUPPORTED, "node %d: conv kernel %dx%d stride %d pad %d unsupported", k, d.kh, d.kw,
                      d.stride, d.pad);
        int ho = (p.h + 2 * d.pad - d.kh) / d.stride + 1;
        int wo = (p.w + 2 * d.pad - d.kw) / d.stride + 1;
        if (ho != d.h || wo != d.w) return fail(VB_ESHAPE, "node %d: conv output %dx%d, expected %dx%d", k, d.h, d.w, ho, wo);
        break;
      }
      case VB_RELU:
        if (d.c != p.c || d.h != p.h || d.w != p.w) return fail(VB_ESHAPE, "node %d: relu shape mismatch", k);
        break;
      case VB_ADD: {
        const NodeInfo& q = G.n[d.in1];
        if (d.c != p.c || d.h != p.h || d.w != p.w || d.c != q.c || d.h != q.h || d.w != q.w)
          return fail(VB_ESHAPE, "node %d: add shape mismatch", k);
        break;
      }
      case VB_GAP:
        if (d.c != p.c || d.h != 1 || d.w != 1) return fail(VB_ESHAPE, "node %d: gap shape mismatch", k);
        break;
      case VB_FLATTEN:
        if (d.size != p.size || d.h != 1 || d.w != 1) return fail(VB_ESHAPE, "node %d: flatten shape mismatch", k);
        break;
      default:
        break;
    }
    G.n[d.in0].cons.push_back(k);
    if (d.op == VB_ADD && d.in1 != d.in0) G.n[d.in1].cons.push_back(k);
  }
  G.L = N - 1;
  return VB_OK;
}

// producer of node k's data, skipping flatten (identity on memory)
int src_of(const Graph& G, int k) {
  while (G.n[k].op == VB_FLATTEN) k = G.n[k].in0;
  return k;
}

// ---------------------------------------------------------------------------
// GEMM descriptors

GemmDesc base_desc() {
  GemmDesc d;
  std::memset(&d, 0, sizeof d);
  d.gh = d.gw = d.hs = d.ws = 1;
  d.sy = d.sx = 1;
  d.ntaps = 1;
  d.ho = d.wo = 1;
  d.oym = d.oxm = 1;
  d.rows_per_b = 1;
  return d;
}

// Dense backward: Psi[rows][n_in] = Lam[rows][n_out] . W[n_out][n_in]
GemmDesc linear_backward(const NodeInfo& nd, const NodeInfo& in, const float* lam, int rows) {
  GemmDesc d = base_desc();
  d.M = rows;
  d.K = (int)nd.size;
  d.N = (int)in.size;
  d.A = lam;
  d.cs = d.K;
  d.a_row_stride = d.K;
  d.B = nd.W;  // replaced by the transposed copy [n_in][n_out]
  return d;
}

// Conv backward for one output-parity class (py, px): Psi over the conv input.
// Returns false if the class has no positions.
bool conv_backward(const NodeInfo& nd, const NodeInfo& in, const float* lam, int rows, int py, int px, GemmDesc& d) {
  d = base_desc();
  const int s = nd.stride, p = nd.pad;
  const int gh = (in.h - py + s - 1) / s, gw = (in.w - px + s - 1) / s;
  if (gh <= 0 || gw <= 0) return false;
  d.gh = gh;
  d.gw = gw;
  d.hs = nd.h;
  d.ws = nd.w;
  d.cs = nd.c;
  d.sy = d.sx = 1;
  d.a_row_stride = nd.size;
  d.ntaps = 0;
  for (int ky = 0; ky < nd.kh; ++ky) {
    if (((py + p - ky) % s + s) % s != 0) continue;
    for (int kx = 0; kx < nd.kw; ++kx) {
      if (((px + p - kx) % s + s) % s != 0) continue;
      d.tap_dy[d.ntaps] = (py + p - ky) / s;  // exact division
      d.tap_dx[d.ntaps] = (px + p - kx) / s;
      d.tap_w[d.ntaps] = ky * nd.kw + kx;
      d.ntaps++;
    }
  }
  d.K = d.ntaps * nd.c;
  d.N = in.c;
  d.M = rows * gh * gw;
  d.A = lam;
  d.B = nd.W;  // replaced by the transposed copy [tap][c_in][c_out]
  d.ho = in.h;
  d.wo = in.w;
  d.oym = s;
  d.oy0 = py;
  d.oxm = s;
  d.ox0 = px;
  return true;
}

// Forward (IBP) affine step of node nd over its producer `in` for `batch` rows.
GemmDesc affine_forward(const NodeInfo& nd, const NodeInfo& in, int batch) {
  GemmDesc d = base_desc();
  if (nd.op == VB_LINEAR) {
    d.M = batch;
    d.K = (int)in.size;
    d.N = nd.c;
    d.cs = d.K;
    d.a_row_stride = d.K;
    d.B = nd.W;  // [n_out][n_in] = [N][K]
    return d;
  }
  d.gh = nd.h;
  d.gw = nd.w;
  d.hs = in.h;
  d.ws = in.w;
  d.cs = in.c;
  d.sy = d.sx = nd.stride;
  d.a_row_stride = in.size;
  d.ntaps = nd.kh * nd.kw;
  for (int ky = 0; ky < nd.kh; ++ky)
    for (int kx = 0; kx < nd.kw; ++kx) {
      int t = ky * nd.kw + kx;
      d.tap_dy[t] = ky - nd.pad;
      d.tap_dx[t] = kx - nd.pad;
      d.tap_w[t] = t;
    }
  d.K = d.ntaps * in.c;
  d.N = nd.c;
  d.M = batch * nd.h * nd.w;
  d.B = nd.W;  // [tap][c_out][c_in] = [tap][N][cs]
  d.ho = nd.h;
  d.wo = nd.w;
  return d;
}

// ---------------------------------------------------------------------------
// backward walk

struct Domain {
  const float* xc;
  const float* xr;
  float eps;
};

struct Backward {
  const Graph& G;
  hipStream_t st;
  const float* const* lo;
  const float* const* hi;
  Domain dom;
  // pool
  float* pool[NPOOL];
  int refs[NPOOL];
  float* part;
  float* rowacc;
  size_t part_floats;
  size_t pool_floats = 0;
  // alpha-CROWN extras (per node, may be NULL)
  const float* const* alpha = nullptr;
  float* const* psi_keep = nullptr;
  // compact alpha / kept Psi of ReLU nodes: column map [batch][size] and row
  // length per node (NULL: [batch][R][size])
  const int* const* aidx = nullptr;
  const int* awidth = nullptr;
  // K-contiguous weight copies for back-substitution, per node
  std::vector<const float*> wt;
  // bias a Lambda over each node carries into beta (ADD nodes: summed over inputs)
  std::vector<const float*> beff;
  // centre / radius of a box domain (stop > 0) for the current chunk
  float* box_c = nullptr;
  float* box_r = nullptr;
  // relaxation coefficients of the current target node, this chunk
  float4* coef = nullptr;
  // optional: return Lambda over the domain node and beta instead of only
  // concretising ([batch][R][size_stop] and [batch][R], whole batch)
  float* a_out = nullptr;
  float* bias_out = nullptr;
  // split constraints of branch-and-bound sub-domains with their multipliers
  // (per ReLU node: split [batch][size], beta [batch][R][size]), or NULL
  const vb_beta* beta = nullptr;
  // selected identity rows over a Linear start (whole batch): neuron lists
  // [batch][n_start], counts [batch], U rows per sign per input
  const int* sel = nullptr;
  const int* cnt = nullptr;
  int U = 0;
  // the current chunk's live-row counts for the GEMMs (selected rows), or NULL
  const int* live_cnt = nullptr;
  int live_u = 0;

  int alloc() {
    for (int i = 0; i < NPOOL; ++i)
      if (refs[i] == 0) {
        refs[i] = 1;
        return i;
      }
    return -1;
  }
  void release(int b) {
    if (b >= 0) refs[b]--;
  }
};

// Bias that a Lambda over node z carries into beta: z's own bias if it is an
// affine node; the sum over both inputs of an ADD (through nested ADDs).
// Returns number of bias vectors written into `out` (up to 4).
void bias_terms(const Graph& G, int z, std::vector<const float*>& out) {
  const NodeInfo& n = G.n[z];
  if (n.op == VB_LINEAR || n.op == VB_CONV2D) {
    if (n.b) out.push_back(n.b);
  } else if (n.op == VB_ADD) {
    bias_terms(G, n.in0, out);
    if (n.in1 != n.in0) bias_terms(G, n.in1, out);
  }
}

// Is node k the lowest-index active consumer of t (through flatten)?
bool lowest_consumer(const Graph& G, const std::vector<char>& active, int t, int k) {
  std::vector<int> stack(G.n[t].cons.begin(), G.n[t].cons.end());
  while (!stack.empty()) {
    int c = stack.back();
    stack.pop_back();
    if (G.n[c].op == VB_FLATTEN) {
      for (int cc : G.n[c].cons) stack.push_back(cc);
      continue;
    }
    if (c != k && active[c] && c < k) return false;
  }
  return true;
}

// Per-chunk parameters of one back-substitution.
struct BwdCall {
  int start, stop;
  const float* C;   // spec rows [chunk][m][n_start] (already offset to the chunk) or NULL: identity
  int m;            // spec rows per batch element (C != NULL)
  int split;        // 1: rows +C and -C (2m rows per element); 0: +C only
  int b0, cb;       // batch offset and chunk size
  int batch_total;
  // selected identity rows (Linear start): neuron list [cb][n_start] and counts
  // [cb] of this chunk, U rows per sign per input; NULL: every neuron
  const int* sel = nullptr;
  const int* cnt = nullptr;
  int U = 0;
};

vb_status effective_bias(Backward& B, const Graph& G, int z, const float*& bias) {
  (void)G;
  bias = B.beff.empty() ? nullptr : B.beff[z];
  return VB_OK;
}

// ---- optional event timing of relaxation-epilogue GEMM launches
struct ProfRec {
  hipEvent_t a, b;
  double flops;
  int32_t info[6];  // epilogue, footprint windows, M, N, K, taps
};
struct ProfDone {
  double ms, flops;
  int32_t info[6];
};
bool g_prof_on = false;
std::vector<ProfRec> g_prof;
std::vector<ProfDone> g_prof_done;  // per launch, from the last vb_profile_stop

vb_status run_gemm_reduce(Backward& B, GemmDesc& d, int rows, int P, bool reduce, double alg_flops = 0.0) {
  d.part = reduce ? B.part : nullptr;
  d.live_cnt = B.live_cnt;
  d.live_u = B.live_u;
  d.part_ld = gemm_ntiles(d);
  if (reduce && (size_t)d.M * d.part_ld > B.part_floats)
    return fail(VB_ENOMEM, "internal: partial buffer too small (%lld > %zu)", (long long)d.M * d.part_ld, B.part_floats);
  const bool prof = g_prof_on && alg_flops > 0.0;
  ProfRec rec{};
  if (prof) {
    HIPCHK(hipEventCreate(&rec.a));
    HIPCHK(hipEventCreate(&rec.b));
    HIPCHK(hipEventRecord(rec.a, B.st));
  }
  HIPCHK(launch_gemm(d, B.st));
  if (prof) {
    HIPCHK(hipEventRecord(rec.b, B.st));
    rec.flops = alg_flops;
    const int32_t info[6] = {d.epi, d.patch, d.M, d.N, d.K, d.ntaps};
    for (int i = 0; i < 6; ++i) rec.info[i] = info[i];
    g_prof.push_back(rec);
  }
  const bool gather = !gemm_is_dense(d);
  if (reduce)
    HIPCHK(launch_rows_reduce(B.part, 1, rows, P, d.part_ld, d.part_ld, B.rowacc, 1, gather ? 1 : 0, B.st));
  return VB_OK;
}

// The output-parity classes of one transposed convolution as one grid, with one
// row reduction over all their positions (class c's partials follow class c-1's
// in the position-major partial buffer).  `joint` comes back false, with
// nothing launched, when the classes do not share a tile shape.
vb_status run_gemm_multi_reduce(Backward& B, std::vector<GemmDesc>& ds, int rows, bool reduce, double alg_flops,
                                bool& joint) {
  const int n = (int)ds.size();
  if (n < 2 || n > MAX_GEMM_MULTI) {
    joint = false;
    return VB_OK;
  }
  const int ld = gemm_ntiles(ds[0]);
  long long P = 0;
  for (GemmDesc& d : ds) {
    if (gemm_ntiles(d) != ld) {
      joint = false;
      return VB_OK;
    }
    d.part = reduce ? B.part + (size_t)P * rows * ld : nullptr;
    d.live_cnt = B.live_cnt;
    d.live_u = B.live_u;
    d.part_ld = ld;
    P += (long long)d.gh * d.gw;
  }
  if (reduce && (size_t)P * rows * ld > B.part_floats) {
    joint = false;  // (the classes one by one need only their own positions' partials)
    return VB_OK;
  }
  const bool prof = g_prof_on && alg_flops > 0.0;
  ProfRec rec{};
  if (prof) {
    HIPCHK(hipEventCreate(&rec.a));
    HIPCHK(hipEventCreate(&rec.b));
    HIPCHK(hipEventRecord(rec.a, B.st));
  }
  const hipError_t e = launch_gemm_multi(ds.data(), n, B.st);
  if (e == hipErrorNotSupported) {
    if (prof) {
      (void)hipEventDestroy(rec.a);
      (void)hipEventDestroy(rec.b);
    }
    joint = false;
    return VB_OK;
  }
  HIPCHK(e);
  if (prof) {
    HIPCHK(hipEventRecord(rec.b, B.st));
    rec.flops = alg_flops;
    const GemmDesc& d = ds[0];
    const int32_t info[6] = {d.epi, d.patch, d.M, d.N, d.K, d.ntaps};
    for (int i = 0; i < 6; ++i) rec.info[i] = info[i];
    g_prof.push_back(rec);
  }
  if (reduce) HIPCHK(launch_rows_reduce(B.part, 1, rows, (int)P, ld, ld, B.rowacc, 1, 1, B.st));
  return VB_OK;
}

// Window of footprint rows over a node's output: cell (Y, X) of the row of start
// pixel (py, px) is pixel (py*sy + oy + Y, px*sx + ox + X).
struct Win {
  int wh = 0, ww = 0, sy = 1, oy = 0, sx = 1, ox = 0;
  bool set = false;
};

// The window a conv's output window reaches on the conv's input.
Win conv_reach(const NodeInfo& nd, const Win& w) {
  Win r;
  r.wh = (w.wh - 1) * nd.stride + nd.kh;
  r.ww = (w.ww - 1) * nd.stride + nd.kw;
  r.sy = w.sy * nd.stride;
  r.oy = w.oy * nd.stride - nd.pad;
  r.sx = w.sx * nd.stride;
  r.ox = w.ox * nd.stride - nd.pad;
  r.set = true;
  return r;
}

// Bounding box of two windows of one scale; false if the scales differ.
bool win_union(Win& a, const Win& b) {
  if (!a.set) {
    a = b;
    return true;
  }
  if (a.sy != b.sy || a.sx != b.sx) return false;
  const int y0 = std::min(a.oy, b.oy), y1 = std::max(a.oy + a.wh, b.oy + b.wh);
  const int x0 = std::min(a.ox, b.ox), x1 = std::max(a.ox + a.ww, b.ox + b.ww);
  a.oy = y0;
  a.wh = y1 - y0;
  a.ox = x0;
  a.ww = x1 - x0;
  return true;
}

bool same_win(const Win& a, const Win& b) {
  return a.wh == b.wh && a.ww == b.ww && a.sy == b.sy && a.oy == b.oy && a.sx == b.sx && a.ox == b.ox;
}

// Algorithmic multiply-adds of one conv step of window rows: for every row, the
// cells of its window over the conv's output that lie inside the image, times
// the conv's multiply-adds per output cell.
// Multiply-adds of one conv step of footprint rows that can be non-zero: per
// start pixel, the output cells of the conv inside the row's window and the
// image, each through the taps that land inside the conv's input image (in_h x
// in_w; a tap into the zero padding multiplies nothing), x C_out (x C_in by the
// caller).  Separable: the (cell, tap) pairs factor into the two axes.
double window_macs(const NodeInfo& S, const NodeInfo& nd, const Win& w, long long rows_per_pixel, int in_h,
                   int in_w) {
  auto axis = [&](int n_start, int step, int off, int len, int n_out, int n_in, int k) {
    double t = 0.0;
    for (int p = 0; p < n_start; ++p) {
      const int a = std::max(p * step + off, 0), b = std::min(p * step + off + len, n_out);
      for (int o = a; o < b; ++o)
        for (int kk = 0; kk < k; ++kk) {
          const int i = o * nd.stride - nd.pad + kk;
          t += (i >= 0 && i < n_in) ? 1.0 : 0.0;
        }
    }
    return t;
  };
  const double ty = axis(S.h, w.sy, w.oy, w.wh, nd.h, in_h, nd.kh);
  const double tx = axis(S.w, w.sx, w.ox, w.ww, nd.w, in_w, nd.kw);
  return (double)rows_per_pixel * ty * tx * nd.c;  // x C_in by the caller
}

// ---- footprint (patch) back-substitution of identity rows through a chain
// conv -> ReLU -> conv ... down to the domain.  Every row is one neuron
// (b, sign, c) at pixel p of the start node; its Lambda over each earlier node
// is non-zero only on the window of pixels that neuron depends on, so Lambda
// is kept on that window (the same size for every p, not clipped at the image
// border: cells outside the node hold zeros).  Returns false if the call does
// not have that shape or the window would not be smaller than the node.
struct PatchStep {
  int k;          // conv node whose Lambda (over its output window) is pushed
  int t;          // its input node (ReLU output or the domain node)
  int wh, ww;     // window of t
  int sy, oy, sx, ox;  // pixel of t for cell (Y, X) of row p = (py, px): py*sy + oy + Y
};

bool patch_chain_graph(const Graph& G, int start, int stop, std::vector<PatchStep>& steps) {
  steps.clear();
  const NodeInfo& S = G.n[start];
  if (S.op != VB_CONV2D || S.cons.empty()) return false;
  int k = start;
  int wh = 1, ww = 1, sy = 1, oy = 0, sx = 1, ox = 0;  // the start node's own 1 x 1 window
  bool smaller = false;
  for (;;) {
    const NodeInfo& nd = G.n[k];
    if (nd.op != VB_CONV2D) return false;
    const int t = nd.in0;
    const NodeInfo& tn = G.n[t];
    PatchStep ps;
    ps.k = k;
    ps.t = t;
    ps.wh = (wh - 1) * nd.stride + nd.kh;
    ps.ww = (ww - 1) * nd.stride + nd.kw;
    ps.sy = sy * nd.stride;
    ps.oy = oy * nd.stride - nd.pad;
    ps.sx = sx * nd.stride;
    ps.ox = ox * nd.stride - nd.pad;
    if (tn.h <= 1 && tn.w <= 1) return false;
    if (nd.kh < nd.stride || nd.kw < nd.stride) return false;  // window cells no tap reaches
    if (ps.wh > tn.h || ps.ww > tn.w) return false;  // window no smaller than the node
    if (ps.wh < tn.h || ps.ww < tn.w) smaller = true;
    steps.push_back(ps);
    if (t == stop) break;
    if (t < stop || tn.op != VB_RELU || tn.cons.size() != 1) return false;
    const int z = tn.in0;
    if (z <= stop || G.n[z].op != VB_CONV2D || G.n[z].cons.size() != 1) return false;
    k = z;
    wh = ps.wh;
    ww = ps.ww;
    sy = ps.sy;
    oy = ps.oy;
    sx = ps.sx;
    ox = ps.ox;
  }
  return smaller;
}

bool patch_chain(const Backward& B, const BwdCall& c, std::vector<PatchStep>& steps) {
  steps.clear();
  if (c.C || B.a_out || B.alpha || B.psi_keep) return false;
  return patch_chain_graph(B.G, c.start, c.stop, steps);
}

// Per batch element: widest Lambda (floats per row) and partial sums of a
// footprint back-substitution of R identity rows; false if it does not apply.
bool patch_requirements(const Graph& G, int start, int stop, long long R, long long& maxw, long long& part_per_b) {
  std::vector<PatchStep> steps;
  if (!patch_chain_graph(G, start, stop, steps)) return false;
  maxw = G.n[start].c;  // the 1 x 1 windows of the identity rows
  part_per_b = 0;
  int wh = 1, ww = 1;
  for (const PatchStep& ps : steps) {
    const NodeInfo& nd = G.n[ps.k];
    const NodeInfo& tn = G.n[ps.t];
    maxw = std::max(maxw, (long long)ps.wh * ps.ww * tn.c);
    if (ps.t == stop && tn.c <= 8 && nd.kh * nd.kw * tn.c <= 64)
      maxw = std::max(maxw, (long long)wh * ww * nd.kh * nd.kw * tn.c);  // tap-expanded product
    const int bn = tn.c > 64 ? 128 : (tn.c > 32 ? 64 : 32);
    part_per_b = std::max(part_per_b, R * ps.wh * ps.ww * ((tn.c + bn - 1) / bn));
    wh = ps.wh;
    ww = ps.ww;
  }
  return true;
}

vb_status backward_chunk_patch(Backward& B, const BwdCall& c, long long R, const std::vector<PatchStep>& steps) {
  const Graph& G = B.G;
  const NodeInfo& S = G.n[c.start];
  const int rows = (int)(c.cb * R);
  for (int i = 0; i < NPOOL; ++i) B.refs[i] = 0;
  // beta starts at +-bias of the start node; Lambda over its own 1 x 1 window is +-e_c
  const float* bias = nullptr;
  vb_status s = effective_bias(B, G, c.start, bias);
  if (s) return s;
  HIPCHK(launch_identity_bias(c.cb, (int)S.size, bias, S.c, B.rowacc, B.st));
  // a domain node inside the network: its box (centre, radius) for this chunk
  if (c.stop != 0)
    HIPCHK(launch_box_center_radius(B.lo[c.stop] + (long long)c.b0 * G.n[c.stop].size,
                                    B.hi[c.stop] + (long long)c.b0 * G.n[c.stop].size,
                                    (long long)c.cb * G.n[c.stop].size, B.box_c, B.box_r, B.st));
  // the first step (through the start conv, relaxed at the ReLU below it) reads
  // the weights directly when the kernel takes the shape; otherwise the
  // identity rows are written out and multiplied like any other Lambda
  const NodeInfo& t0 = G.n[steps[0].t];
  PatchIdRelax pir{};
  pir.W = S.W;
  pir.Co = S.c;
  pir.Ci = t0.c;
  pir.kh = S.kh;
  pir.kw = S.kw;
  pir.out = nullptr;
  const bool direct_first = steps[0].t != c.stop && patch_id_relax_fits(pir);
  int cur = -1;
  if (!direct_first) {
    cur = B.alloc();
    if (cur < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted");
    HIPCHK(launch_patch_identity(rows, (int)R, S.c, B.pool[cur], B.st));
  }
  int wh = 1, ww = 1;
  int ksy = 1, koy = 0, ksx = 1, kox = 0;  // window geometry of the Lambda being pushed
  for (const PatchStep& ps : steps) {
    const NodeInfo& nd = G.n[ps.k];
    const NodeInfo& tn = G.n[ps.t];
    const bool last = ps.t == c.stop;
    const int z = last ? -1 : tn.in0;
    int outb = -1;
    const float* bias_z = nullptr;
    if (!last) {
      outb = B.alloc();
      if (outb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted");
      s = effective_bias(B, G, z, bias_z);
      if (s) return s;
      HIPCHK(launch_relax_coef(B.lo[z] + (long long)c.b0 * G.n[z].size, B.hi[z] + (long long)c.b0 * G.n[z].size,
                               (long long)c.cb * G.n[z].size, nullptr, B.coef, B.st));
    }
    if (cur < 0) {
      // (direct_first: this is the start conv and not the last step)
      pir.R = (int)R;
      pir.pgh = S.h;
      pir.pgw = S.w;
      pir.psy = ps.sy;
      pir.poy = ps.oy;
      pir.psx = ps.sx;
      pir.pox = ps.ox;
      pir.img_h = tn.h;
      pir.img_w = tn.w;
      pir.coef = B.coef;
      pir.bias = bias_z;
      pir.out = B.pool[outb];
      HIPCHK(launch_patch_id_relax(pir, rows, B.rowacc, B.st));
      cur = outb;
      wh = ps.wh;
      ww = ps.ww;
      ksy = ps.sy;
      koy = ps.oy;
      ksx = ps.sx;
      kox = ps.ox;
      continue;
    }
    if (last) {
      // few domain channels: the direct kernel over each row's window (the
      // transposed conv on matrix blocks and the concretisation in one pass)
      ConvIn a{};
      a.lam = B.pool[cur];
      a.W = nd.W;
      a.Co = nd.c;
      a.Ho = wh;
      a.Wo = ww;
      a.Ci = tn.c;
      a.Hi = ps.wh;
      a.Wi = ps.ww;
      a.kh = nd.kh;
      a.kw = nd.kw;
      a.stride = nd.stride;
      a.pad = 0;  // the window covers every tap
      a.rows_per_b = (int)R;
      if (c.stop == 0) {
        a.center = B.dom.xc + (long long)c.b0 * G.n[0].size;
        a.radius = B.dom.xr ? B.dom.xr + (long long)c.b0 * G.n[0].size : nullptr;
        a.eps = B.dom.eps;
      } else {
        a.center = B.box_c;
        a.radius = B.box_r;
      }
      a.patch = 1;
      a.pc = S.c;
      a.pgh = S.h;
      a.pgw = S.w;
      a.psy = ps.sy;
      a.poy = ps.oy;
      a.psx = ps.sx;
      a.pox = ps.ox;
      a.img_h = tn.h;
      a.img_w = tn.w;
      if (conv_input_fits(a) && conv_input_part_floats(a, rows) <= B.part_floats) {
        HIPCHK(launch_conv_input_concretize(a, rows, B.part, B.rowacc, B.st));
        B.release(cur);
        break;
      }
    }
    if (last && tn.c <= 8 && nd.kh * nd.kw * tn.c <= 64 &&
        (size_t)rows * wh * ww * nd.kh * nd.kw * tn.c <= B.pool_floats) {
      // few domain channels: Q = Lambda . W over (tap, c_in) columns as a dense
      // GEMM, then the taps are summed per window cell and concretised
      const int qb = B.alloc();
      if (qb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted");
      GemmDesc d = base_desc();
      d.M = rows * wh * ww;
      d.K = nd.c;
      d.N = nd.kh * nd.kw * tn.c;
      d.cs = d.K;
      d.a_row_stride = d.K;
      d.A = B.pool[cur];
      d.B = B.wt[ps.k];
      d.epi = E_STORE;
      d.out = B.pool[qb];
      s = run_gemm_reduce(B, d, rows, 1, false, 2.0 * d.M * d.N * d.K);
      if (s) return s;
      Col2Im a{};
      a.Q = B.pool[qb];
      a.Ho = wh;
      a.Wo = ww;
      a.Ci = tn.c;
      a.Hi = ps.wh;
      a.Wi = ps.ww;
      a.kh = nd.kh;
      a.kw = nd.kw;
      a.stride = nd.stride;
      a.pad = 0;
      a.rows_per_b = (int)R;
      a.mode = E_CONCRETIZE;
      if (c.stop == 0) {
        a.center = B.dom.xc + (long long)c.b0 * G.n[0].size;
        a.radius = B.dom.xr ? B.dom.xr + (long long)c.b0 * G.n[0].size : nullptr;
        a.eps = B.dom.eps;
      } else {
        a.center = B.box_c;
        a.radius = B.box_r;
      }
      a.patch = 1;
      a.pc = S.c;
      a.pgh = S.h;
      a.pgw = S.w;
      a.psy = ps.sy;
      a.poy = ps.oy;
      a.psx = ps.sx;
      a.pox = ps.ox;
      a.img_h = tn.h;
      a.img_w = tn.w;
      HIPCHK(launch_col2im(a, rows, B.rowacc, B.st));
      B.release(qb);
      B.release(cur);
      break;
    }
    // the conv as a transposed conv between windows: output window wh x ww of k,
    // input window ps.wh x ps.ww of t, no padding (the window covers every tap)
    NodeInfo nv = nd, tv = tn;
    nv.h = wh;
    nv.w = ww;
    nv.pad = 0;
    nv.size = (long long)wh * ww * nd.c;
    tv.h = ps.wh;
    tv.w = ps.ww;
    tv.size = (long long)ps.wh * ps.ww * tn.c;
    for (int py = 0; py < nd.stride; ++py)
      for (int px = 0; px < nd.stride; ++px) {
        GemmDesc d;
        if (!conv_backward(nv, tv, B.pool[cur], rows, py, px, d)) continue;
        if (d.K == 0) continue;  // (excluded by patch_chain: kh, kw >= stride)
        d.B = B.wt[ps.k];
        d.coef = B.coef;
        d.rows_per_b = (int)R;
        d.patch = 1;
        d.pc = S.c;
        d.pgh = S.h;
        d.pgw = S.w;
        d.psy = ps.sy;
        d.poy = ps.oy;
        d.psx = ps.sx;
        d.pox = ps.ox;
        d.img_h = tn.h;
        d.img_w = tn.w;
        d.ssy = ksy;
        d.soy = koy;
        d.ssx = ksx;
        d.sox = kox;
        d.src_h = nd.h;
        d.src_w = nd.w;
        if (last) {
          d.epi = E_CONCRETIZE;
          if (c.stop == 0) {
            d.center = B.dom.xc + (long long)c.b0 * G.n[0].size;
            d.radius = B.dom.xr ? B.dom.xr + (long long)c.b0 * G.n[0].size : nullptr;
            d.eps = B.dom.eps;
          } else {
            d.center = B.box_c;
            d.radius = B.box_r;
          }
        } else {
          d.epi = E_RELAX;
          d.out = B.pool[outb];
          d.bias = bias_z;
          d.bias_c = tn.c;
        }
        // (profiled work: the multiply-adds of the rows' window cells inside the
        // image through taps inside the input image, except the first step from
        // the identity rows, which is a copy of the weight footprint)
        const double macs = ps.k == c.start ? 0.0
                                            : window_macs(S, nd, Win{wh, ww, ksy, koy, ksx, kox, true},
                                                          (long long)c.cb * 2 * S.c, tn.h, tn.w) * tn.c;
        s = run_gemm_reduce(B, d, rows, d.gh * d.gw, true, 2.0 * macs / (nd.stride * nd.stride));
        if (s) return s;
      }
    B.release(cur);
    cur = outb;
    wh = ps.wh;
    ww = ps.ww;
    ksy = ps.sy;
    koy = ps.oy;
    ksx = ps.sx;
    kox = ps.ox;
  }
  return VB_OK;
}

// ---- footprint (window) back-substitution of identity rows through a region
// of Conv / ReLU / ADD nodes (residual blocks).  Every row is one neuron (b,
// sign, c) at pixel p of the start node, as in the chain case; its Lambda over
// each node of the region is kept on a window of that node's output: the
// bounding box of what reaches the node from the start pixel along every path
// (for a residual block, the union of the convolution branch and the skip).
// All rows share the window's size; cell (Y, X) of the row of pixel (py, px)
// is pixel (py*sy + oy + Y, px*sx + ox + X), cells outside the image hold
// zeros.  A conv step is a transposed convolution from the conv's output
// window to its input's window; a branch that reaches the domain node is
// concretised there over its own reach, so the branches are summed in beta
// and never need a common window at the domain.
// Windows of identity rows over `start` on every node down to `stop` (the
// domain node itself gets none: each branch reaching it is concretised on its
// own reach).  Applies to regions whose nodes are Conv, ReLU and ADD (with at
// least one ADD: plain conv chains take the chain walker) where every ReLU's
// lowest active consumer is a Conv that can fuse the relaxation (its input
// feeding only that ReLU), every Conv reaches a ReLU or the domain, and no
// window is as large as its node.  `active` receives the nodes reached.
bool window_plan(const Graph& G, int start, int stop, std::vector<Win>& W, std::vector<char>& active) {
  const int N = (int)G.n.size();
  const NodeInfo& S = G.n[start];
  if ((S.op != VB_CONV2D && S.op != VB_ADD) || S.h * S.w <= 1) return false;
  W.assign(N, Win{});
  active.assign(N, 0);
  W[start] = Win{1, 1, 1, 0, 1, 0, true};
  bool has_add = false, smaller = false;
  for (int k = start; k > stop; --k) {
    if (!W[k].set) continue;
    active[k] = 1;
    const NodeInfo& nd = G.n[k];
    Win w = W[k];
    if (nd.op == VB_CONV2D) {
      w = conv_reach(nd, w);  // (a kernel smaller than its stride: only onto the domain, checked below)
    } else if (nd.op == VB_ADD) {
      has_add = true;
      if (nd.in0 == nd.in1) return false;
    } else if (nd.op != VB_RELU) {
      return false;
    }
    const int ins[2] = {nd.in0, nd.op == VB_ADD ? nd.in1 : -1};
    for (int q = 0; q < 2; ++q) {
      const int t = ins[q];
      if (t < 0) continue;
      if (t < stop || G.n[t].h * G.n[t].w <= 1) return false;
      if (t == stop) {
        if (nd.op != VB_CONV2D) return false;  // only a conv step concretises onto the domain
        active[t] = 1;
        if (!win_union(W[t], w)) return false;  // several branches are summed there first
        continue;
      }
      if (!win_union(W[t], w)) return false;
    }
  }
  if (!has_add) return false;
  for (int k = stop + 1; k <= start; ++k) {
    if (!active[k]) continue;
    const NodeInfo& nd = G.n[k];
    if (W[k].wh > nd.h || W[k].ww > nd.w) return false;
    if (W[k].wh < nd.h || W[k].ww < nd.w) smaller = true;
    if (nd.op == VB_RELU) {
      // the lowest active consumer relaxes: a conv whose input is this ReLU, and the
      // ReLU's input feeds nothing else
      int low = -1;
      for (int c : nd.cons)
        if (active[c] && (low < 0 || c < low)) low = c;
      if (low < 0 || G.n[low].op != VB_CONV2D || G.n[nd.in0].cons.size() != 1) return false;
      if (!same_win(W[k], W[nd.in0])) return false;
    }
    if (nd.op == VB_CONV2D) {
      const int t = nd.in0;
      if (t != stop && G.n[t].op != VB_RELU) return false;
      if (t != stop) {
        int low = -1;
        for (int c : G.n[t].cons)
          if (active[c] && (low < 0 || c < low)) low = c;
        if (low != k) return false;  // (another conv relaxes there: would need a stored product)
        // every output-parity class of the transposed conv must have a tap
        if (nd.kh < nd.stride || nd.kw < nd.stride) return false;
      }
    }
    if (nd.op == VB_ADD) {
      for (int t : {nd.in0, nd.in1})
        if (t != stop && G.n[t].op != VB_CONV2D && G.n[t].op != VB_RELU) return false;
    }
  }
  return smaller;
}

// Per batch element: widest window (floats per row) and partial sums of a
// window back-substitution of R identity rows; false if it does not apply.
bool window_requirements(const Graph& G, int start, int stop, long long R, long long& maxw, long long& part_per_b) {
  std::vector<Win> W;
  std::vector<char> active;
  if (!window_plan(G, start, stop, W, active)) return false;
  maxw = G.n[start].c;
  part_per_b = 0;
  for (int k = stop + 1; k <= start; ++k) {
    if (!active[k]) continue;
    const NodeInfo& nd = G.n[k];
    maxw = std::max(maxw, (long long)W[k].wh * W[k].ww * nd.c);
    if (nd.op == VB_CONV2D) {
      const NodeInfo& tn = G.n[nd.in0];
      const Win tw = nd.in0 == stop ? conv_reach(nd, W[k]) : W[nd.in0];
      const int bn = tn.c > 64 ? 128 : (tn.c > 32 ? 64 : 32);
      part_per_b = std::max(part_per_b, R * tw.wh * tw.ww * ((tn.c + bn - 1) / bn));
      if (nd.in0 == stop || k == start) maxw = std::max(maxw, (long long)tw.wh * tw.ww * tn.c);
    }
  }
  // branches meeting at the domain node are summed on its window first
  maxw = std::max(maxw, (long long)W[stop].wh * W[stop].ww * G.n[stop].c);
  const int bn = G.n[stop].c > 64 ? 128 : (G.n[stop].c > 32 ? 64 : 32);
  part_per_b = std::max(part_per_b, R * W[stop].wh * W[stop].ww * ((G.n[stop].c + bn - 1) / bn));
  return true;
}

vb_status backward_chunk_window(Backward& B, const BwdCall& c, long long R, const std::vector<Win>& W,
                                const std::vector<char>& active) {
  const Graph& G = B.G;
  const NodeInfo& S = G.n[c.start];
  const int N = (int)G.n.size();
  const int rows = (int)(c.cb * R);
  for (int i = 0; i < NPOOL; ++i) B.refs[i] = 0;
  // pending Lambda per node: a pool buffer in window geometry pw[k], or IDENT
  // (the identity rows themselves, over a node one ADD below the start)
  constexpr int NONE = -1, IDENT_ROWS = -2;
  std::vector<int> lam(N, NONE);
  std::vector<Win> pw(N);
  const float* bias = nullptr;
  vb_status s = effective_bias(B, G, c.start, bias);
  if (s) return s;
  HIPCHK(launch_identity_bias(c.cb, (int)S.size, bias, S.c, B.rowacc, B.st));
  if (c.stop != 0)
    HIPCHK(launch_box_center_radius(B.lo[c.stop] + (long long)c.b0 * G.n[c.stop].size,
                                    B.hi[c.stop] + (long long)c.b0 * G.n[c.stop].size,
                                    (long long)c.cb * G.n[c.stop].size, B.box_c, B.box_r, B.st));
  const Win one{1, 1, 1, 0, 1, 0, true};
  if (S.op == VB_ADD) {
    lam[S.in0] = lam[S.in1] = IDENT_ROWS;
    pw[S.in0] = pw[S.in1] = one;
  } else {
    lam[c.start] = IDENT_ROWS;
    pw[c.start] = one;
  }
  const long long rows_per_pixel = (long long)c.cb * 2 * S.c;
  auto chunk_off = [&](int node) -> long long { return (long long)c.b0 * G.n[node].size; };
  // Branches that reach the domain node: the bound is min over the box of the SUM
  // of their Lambdas (|L1 + L2| <= |L1| + |L2|), so all but the last one store
  // their product on the domain's window (the union of the branches' reaches) and
  // the last one concretises that sum.  (One branch: it concretises on its reach.)
  int dom_edges = 0, last_edge = -1;
  for (int k = c.stop + 1; k <= c.start; ++k)
    if (active[k] && G.n[k].op == VB_CONV2D && G.n[k].in0 == c.stop) {
      ++dom_edges;
      if (last_edge < 0) last_edge = k;
    }
  int dom_buf = -1;
  // Two conv branches onto the domain with the same stride and number of output
  // channels are concretised by ONE GEMM whose taps read both branches' Lambdas
  // (the K loop runs over the taps of both), so the sum is formed in the
  // accumulators: no domain-window buffer to clear, store and read back.  The
  // first of the two branches the walk meets waits for the second.
  bool merge_dom = false;
  if (dom_edges == 2) {
    int e[2], n = 0;
    for (int k = c.stop + 1; k <= c.start; ++k)
      if (active[k] && G.n[k].op == VB_CONV2D && G.n[k].in0 == c.stop) e[n++] = k;
    const NodeInfo &a = G.n[e[0]], &b = G.n[e[1]];
    const auto per_class = [](const NodeInfo& q) {
      return ((q.kh + q.stride - 1) / q.stride) * ((q.kw + q.stride - 1) / q.stride);
    };
    merge_dom = a.stride == b.stride && a.c == b.c && a.c % 32 == 0 && per_class(a) + per_class(b) <= MAX_TAPS;
  }
  struct Deferred {
    int k = -1, buf = -1;
    Win w;
  } held;
  // a pool buffer holding the pending Lambda of node t in window geometry w
  auto as_buffer = [&](int t, const Win& w, int& out) -> vb_status {
    out = B.alloc();
    if (out < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", t);
    const Win& g = pw[t];
    const int oy = g.oy - w.oy, ox = g.ox - w.ox;
    if (g.sy != w.sy || g.sx != w.sx || oy < 0 || ox < 0 || oy + g.wh > w.wh || ox + g.ww > w.ww)
      return fail(VB_EUNSUPPORTED, "internal: window of node %d does not contain its pending Lambda", t);
    if (lam[t] == IDENT_ROWS) {
      HIPCHK(launch_window_identity(rows, (int)R, S.c, w.wh, w.ww, oy, ox, B.pool[out], B.st));
    } else {
      HIPCHK(launch_window_embed(B.pool[lam[t]], rows, G.n[t].c, g.wh, g.ww, w.wh, w.ww, oy, ox, B.pool[out],
                                 B.st));
      B.release(lam[t]);
    }
    lam[t] = NONE;
    return VB_OK;
  };
  auto patch_fields = [&](GemmDesc& d, const Win& out_w, const NodeInfo& tn, const Win& src_w, const NodeInfo& kn) {
    d.rows_per_b = (int)R;
    d.patch = 1;
    d.pc = S.c;
    d.pgh = S.h;
    d.pgw = S.w;
    d.psy = out_w.sy;
    d.poy = out_w.oy;
    d.psx = out_w.sx;
    d.pox = out_w.ox;
    d.img_h = tn.h;
    d.img_w = tn.w;
    d.ssy = src_w.sy;
    d.soy = src_w.oy;
    d.ssx = src_w.sx;
    d.sox = src_w.ox;
    d.src_h = kn.h;
    d.src_w = kn.w;
  };
  for (int k = c.start; k > c.stop; --k) {
    if (!active[k] || lam[k] == NONE) continue;
    const NodeInfo& nd = G.n[k];
    if (nd.op == VB_ADD) {
      // Lambda over an ADD flows unchanged into both inputs (window of the ADD)
      if (lam[k] == IDENT_ROWS) return fail(VB_EUNSUPPORTED, "internal: identity rows over a nested ADD");
      for (int t : {nd.in0, nd.in1}) {
        if (lam[t] != NONE) return fail(VB_EUNSUPPORTED, "internal: two Lambdas meet at node %d", t);
        B.refs[lam[k]]++;
        lam[t] = lam[k];
        pw[t] = pw[k];
      }
      B.release(lam[k]);
      lam[k] = NONE;
      continue;
    }
    if (nd.op != VB_CONV2D) return fail(VB_EUNSUPPORTED, "internal: window rows pending at node %d", k);
    const int t = nd.in0;
    const NodeInfo& tn = G.n[t];
    const bool last = t == c.stop;
    const int z = last ? -1 : tn.in0;
    // the first step of identity rows through a conv whose input ReLU relaxes:
    // a relaxed copy of the weight footprint, no GEMM
    if (lam[k] == IDENT_ROWS && !last && lam[t] == NONE && same_win(conv_reach(nd, one), W[t])) {
      PatchIdRelax pir{};
      pir.W = nd.W;
      pir.Co = nd.c;
      pir.Ci = tn.c;
      pir.kh = nd.kh;
      pir.kw = nd.kw;
      if (patch_id_relax_fits(pir) && nd.c == S.c && nd.h == S.h && nd.w == S.w) {
        const float* bias_z = nullptr;
        if ((s = effective_bias(B, G, z, bias_z))) return s;
        HIPCHK(launch_relax_coef(B.lo[z] + chunk_off(z), B.hi[z] + chunk_off(z), (long long)c.cb * G.n[z].size,
                                 nullptr, B.coef, B.st));
        const int outb = B.alloc();
        if (outb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
        pir.R = (int)R;
        pir.pgh = S.h;
        pir.pgw = S.w;
        pir.psy = W[t].sy;
        pir.poy = W[t].oy;
        pir.psx = W[t].sx;
        pir.pox = W[t].ox;
        pir.img_h = tn.h;
        pir.img_w = tn.w;
        pir.coef = B.coef;
        pir.bias = bias_z;
        pir.out = B.pool[outb];
        HIPCHK(launch_patch_id_relax(pir, rows, B.rowacc, B.st));
        lam[k] = NONE;
        lam[z] = outb;
        pw[z] = W[t];
        continue;
      }
    }
    int cur;
    if (lam[k] == IDENT_ROWS) {
      // identity rows over this conv's output, one-hot on a 1 x 1 window
      if ((s = as_buffer(k, one, cur))) return s;
    } else {
      cur = lam[k];
      lam[k] = NONE;
    }
    const Win kw = pw[k];
    const bool summed = last && dom_edges > 1 && !merge_dom;
    const Win tw = last ? (dom_edges > 1 ? W[t] : conv_reach(nd, kw)) : W[t];
    if (last && merge_dom && k != last_edge) {
      held.k = k;
      held.buf = cur;
      held.w = kw;
      continue;
    }
    int outb = -1, addb = -1;
    const float* bias_z = nullptr;
    if (summed && dom_buf < 0) {
      dom_buf = B.alloc();
      if (dom_buf < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
      HIPCHK(launch_fill(B.pool[dom_buf], 0.f, (long long)rows * tw.wh * tw.ww * tn.c, B.st));
    }
    if (!last) {
      if (lam[t] >= 0 && same_win(pw[t], tw)) {
        addb = lam[t];  // already in the target's window: added as it is
        lam[t] = NONE;
      } else if (lam[t] != NONE && (s = as_buffer(t, tw, addb))) {
        return s;
      }
      outb = B.alloc();
      if (outb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
      if ((s = effective_bias(B, G, z, bias_z))) return s;
      HIPCHK(launch_relax_coef(B.lo[z] + chunk_off(z), B.hi[z] + chunk_off(z), (long long)c.cb * G.n[z].size,
                               nullptr, B.coef, B.st));
    }
    // the conv as a transposed conv from window kw to window tw: target cell
    // Yt = stride * Yk + ky - pad_eff with pad_eff = pad + oy_t - stride * oy_k
    NodeInfo nv = nd, tv = tn;
    nv.h = kw.wh;
    nv.w = kw.ww;
    nv.size = (long long)kw.wh * kw.ww * nd.c;
    tv.h = tw.wh;
    tv.w = tw.ww;
    tv.size = (long long)tw.wh * tw.ww * tn.c;
    const int pad_y = nd.pad + tw.oy - nd.stride * kw.oy, pad_x = nd.pad + tw.ox - nd.stride * kw.ox;
    if (pad_y != pad_x) return fail(VB_EUNSUPPORTED, "internal: windows of node %d are not square-aligned", k);
    nv.pad = pad_y;
    // the multiply-adds of this step (cells of the rows' windows inside the image,
    // taps inside the input image)
    const double macs = window_macs(S, nd, kw, rows_per_pixel, tn.h, tn.w) * tn.c;
    double macs_all = macs;
    std::vector<GemmDesc> descs;
    if (last && merge_dom) {
      if (held.k < 0) return fail(VB_EUNSUPPORTED, "internal: the other branch onto node %d is missing", t);
      const NodeInfo& nd1 = G.n[held.k];
      const Win& kw1 = held.w;
      NodeInfo nv1 = nd1;
      nv1.h = kw1.wh;
      nv1.w = kw1.ww;
      nv1.size = (long long)kw1.wh * kw1.ww * nd1.c;
      nv1.pad = nd1.pad + tw.oy - nd1.stride * kw1.oy;
      if (nv1.pad != nd1.pad + tw.ox - nd1.stride * kw1.ox)
        return fail(VB_EUNSUPPORTED, "internal: windows of node %d are not square-aligned", held.k);
      macs_all += window_macs(S, nd1, kw1, rows_per_pixel, tn.h, tn.w) * tn.c;
      for (int py = 0; py < nd.stride; ++py)
        for (int px = 0; px < nd.stride; ++px) {
          GemmDesc d0, d1;
          const bool h0 = conv_backward(nv, tv, B.pool[cur], rows, py, px, d0) && d0.K > 0;
          const bool h1 = conv_backward(nv1, tv, B.pool[held.buf], rows, py, px, d1) && d1.K > 0;
          if (!h0 && !h1) continue;
          GemmDesc d = h0 ? d0 : d1;
          d.B = h0 ? B.wt[k] : B.wt[held.k];
          patch_fields(d, tw, tn, h0 ? kw : kw1, h0 ? nd : nd1);
          if (h0 && h1) {
            if (d1.gh != d.gh || d1.gw != d.gw || d1.oy0 != d.oy0 || d1.ox0 != d.ox0 || d1.cs != d.cs ||
                d.ntaps + d1.ntaps > MAX_TAPS)
              return fail(VB_EUNSUPPORTED, "internal: the branches onto node %d do not share their grid", t);
            d.tap_src1 = d.ntaps;
            for (int j = 0; j < d1.ntaps; ++j) {
              d.tap_dy[d.ntaps + j] = d1.tap_dy[j];
              d.tap_dx[d.ntaps + j] = d1.tap_dx[j];
              d.tap_w[d.ntaps + j] = d1.tap_w[j];
            }
            d.ntaps += d1.ntaps;
            d.K = d.ntaps * d.cs;
            d.A1 = B.pool[held.buf];
            d.B1 = B.wt[held.k];
            d.a1_row_stride = d1.a_row_stride;
            d.hs1 = d1.hs;
            d.ws1 = d1.ws;
            d.ssy1 = kw1.sy;
            d.soy1 = kw1.oy;
            d.ssx1 = kw1.sx;
            d.sox1 = kw1.ox;
            d.src_h1 = nd1.h;
            d.src_w1 = nd1.w;
          }
          descs.push_back(d);
        }
    } else {
      for (int py = 0; py < nd.stride; ++py)
        for (int px = 0; px < nd.stride; ++px) {
          GemmDesc d;
          if (conv_backward(nv, tv, B.pool[cur], rows, py, px, d) && d.K > 0) {
            d.B = B.wt[k];
            patch_fields(d, tw, tn, kw, nd);
            descs.push_back(d);
          }
        }
    }
    for (GemmDesc& d : descs) {
      if (summed && k != last_edge) {
        // a branch onto the domain that is not the last: add into the domain window
        d.epi = E_STORE;
        d.out = B.pool[dom_buf];
        d.addend = B.pool[dom_buf];
      } else if (last) {
        d.epi = E_CONCRETIZE;
        d.addend = summed ? B.pool[dom_buf] : nullptr;
        if (c.stop == 0) {
          d.center = B.dom.xc + chunk_off(0);
          d.radius = B.dom.xr ? B.dom.xr + chunk_off(0) : nullptr;
          d.eps = B.dom.eps;
        } else {
          d.center = B.box_c;
          d.radius = B.box_r;
        }
      } else {
        d.epi = E_RELAX;
        d.coef = B.coef;
        d.out = B.pool[outb];
        d.addend = addb >= 0 ? B.pool[addb] : nullptr;
        d.bias = bias_z;
        d.bias_c = tn.c;
      }
      s = run_gemm_reduce(B, d, rows, d.gh * d.gw, d.epi != E_STORE, 2.0 * macs_all / descs.size());
      if (s) return s;
    }
    if (!last && descs.size() != (size_t)nd.stride * nd.stride)
      return fail(VB_EUNSUPPORTED, "internal: node %d has output-parity classes without taps", k);
    B.release(cur);
    if (last && merge_dom) {
      B.release(held.buf);
      held = Deferred{};
    }
    if (addb >= 0) B.release(addb);
    if (summed && k == last_edge) {
      B.release(dom_buf);
      dom_buf = -1;
    }
    if (!last) {
      lam[z] = outb;
      pw[z] = tw;
    }
  }
  return VB_OK;
}

// Lambda over a conv's few-channel domain node concretised in one direct
// kernel (no tap-expanded product in between).  `done` stays false (nothing
// launched) if the kernel does not take the shape.  (Not a GEMM: it is not
// recorded by the GEMM profile.)
vb_status direct_conv_input(Backward& B, const NodeInfo& nd, const NodeInfo& tn, int t, int rows, int cur, int pbuf,
                            const BwdCall& c, bool& done) {
  done = false;
  ConvIn a{};
  a.lam = B.pool[cur];
  a.W = nd.W;
  a.Co = nd.c;
  a.Ho = nd.h;
  a.Wo = nd.w;
  a.Ci = tn.c;
  a.Hi = tn.h;
  a.Wi = tn.w;
  a.kh = nd.kh;
  a.kw = nd.kw;
  a.stride = nd.stride;
  a.pad = nd.pad;
  const long long R = rows / c.cb;
  a.rows_per_b = (int)R;
  if (!conv_input_fits(a) || conv_input_part_floats(a, rows) > B.part_floats) return VB_OK;
  a.addend = pbuf >= 0 ? B.pool[pbuf] : nullptr;
  a.psi_out = (B.psi_keep && B.psi_keep[t]) ? B.psi_keep[t] + (long long)c.b0 * R * tn.size : nullptr;
  if (t == 0) {
    a.center = B.dom.xc + (long long)c.b0 * tn.size;
    a.radius = B.dom.xr ? B.dom.xr + (long long)c.b0 * tn.size : nullptr;
    a.eps = B.dom.eps;
  } else {
    a.center = B.box_c;
    a.radius = B.box_r;
  }
  HIPCHK(launch_conv_input_concretize(a, rows, B.part, B.rowacc, B.st));
  done = true;
  return VB_OK;
}

// Execute the back-substitution of call `c`; rowacc receives the lower bound
// of every row (rows = cb * R).  Lambda of a node is a pool buffer, or IDENT:
// the implicit +-I over the start node (identity rows), which Linear and Conv
// nodes consume through footprint kernels instead of a GEMM over an identity.
constexpr int IDENT = -2;

vb_status backward_chunk(Backward& B, const BwdCall& c, long long R) {
  {
    std::vector<PatchStep> steps;
    if (patch_chain(B, c, steps)) return backward_chunk_patch(B, c, R, steps);
    std::vector<Win> W;
    std::vector<char> act;
    if (!(c.C || B.a_out || B.alpha || B.psi_keep) && window_plan(B.G, c.start, c.stop, W, act))
      return backward_chunk_window(B, c, R, W, act);
  }
  const Graph& G = B.G;
  const int N = (int)G.n.size();
  const int rows = (int)(c.cb * R);
  std::vector<int> lam(N, -1);
  for (int i = 0; i < NPOOL; ++i) B.refs[i] = 0;

  // active nodes: reachable backwards from start without passing below stop
  std::vector<char> active(N, 0);
  {
    std::vector<int> stack{c.start};
    while (!stack.empty()) {
      int k = stack.back();
      stack.pop_back();
      if (active[k]) continue;
      active[k] = 1;
      if (k == c.stop) continue;
      if (k == 0) return fail(VB_ESHAPE, "node %d is not bounded by domain node %d", c.start, c.stop);
      stack.push_back(G.n[k].in0);
      if (G.n[k].op == VB_ADD) stack.push_back(G.n[k].in1);
    }
    if (!active[c.stop]) return fail(VB_ESHAPE, "domain node %d does not feed node %d", c.start, c.stop);
    for (int k = 0; k < c.stop; ++k) active[k] = 0;
  }
  auto chunk_off = [&](int node) -> long long { return (long long)c.b0 * G.n[node].size; };
  // per-row tensors over a node (alpha, kept Psi: [batch][R][size]) for this chunk
  // (compact ReLU state: rows of awidth[node] columns)
  auto compact = [&](int node) { return B.aidx && G.n[node].op == VB_RELU; };
  auto row_off = [&](int node) -> long long {
    return (long long)c.b0 * R * (compact(node) ? (long long)B.awidth[node] : G.n[node].size);
  };
  auto alpha_of = [&](int node) -> const float* {
    return (B.alpha && B.alpha[node]) ? B.alpha[node] + row_off(node) : nullptr;
  };
  auto psi_of = [&](int node) -> float* {
    return (B.psi_keep && B.psi_keep[node]) ? B.psi_keep[node] + row_off(node) : nullptr;
  };
  auto aidx_of = [&](int node) -> const int* { return compact(node) ? B.aidx[node] + chunk_off(node) : nullptr; };
  auto acols_of = [&](int node) -> int { return compact(node) ? B.awidth[node] : 0; };
  const NodeInfo& S = G.n[c.start];
  if (c.stop != 0)
    HIPCHK(launch_box_center_radius(B.lo[c.stop] + chunk_off(c.stop), B.hi[c.stop] + chunk_off(c.stop),
                                    (long long)c.cb * G.n[c.stop].size, B.box_c, B.box_r, B.st));

  // materialise the implicit identity of node k (dense +-I rows over it)
  auto materialise = [&](int k) -> vb_status {
    int b = B.alloc();
    if (b < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
    HIPCHK(launch_identity_fill(c.cb, (int)S.size, B.pool[b], B.st));
    lam[k] = b;
    return VB_OK;
  };
  // accumulate a buffer into node t's pending Lambda (takes over one reference of `buf`)
  auto accumulate = [&](int t, int buf) -> vb_status {
    if (lam[t] == -1) {
      lam[t] = buf;
      return VB_OK;
    }
    if (lam[t] == IDENT) {
      vb_status s = materialise(t);
      if (s) return s;
    }
    int outb = B.refs[lam[t]] == 1 ? lam[t] : B.alloc();
    if (outb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", t);
    HIPCHK(launch_add(B.pool[lam[t]], B.pool[buf], 1.f, B.pool[outb], (long long)rows * G.n[t].size, B.st));
    if (outb != lam[t]) B.release(lam[t]);
    B.release(buf);
    lam[t] = outb;
    return VB_OK;
  };

  int from = c.start;
  if (c.C) {
    int b = B.alloc();
    const float* bias = nullptr;
    vb_status s = effective_bias(B, G, c.start, bias);
    if (s) return s;
    HIPCHK(launch_spec_init(c.C, c.cb, c.m, (int)S.size, bias, S.c, B.pool[b], B.rowacc, c.split, B.st));
    lam[c.start] = b;
  } else {
    const float* bias = nullptr;
    vb_status s = effective_bias(B, G, c.start, bias);
    if (s) return s;
    // fast path: Linear start whose input is a ReLU -> relaxed rows of +-W in one kernel
    // (with alpha slopes or kept Psi the identity rows go through the GEMM
    // epilogues, which apply them; the fused first-step kernels do not)
    int t = (S.op == VB_LINEAR && !B.alpha && !B.psi_keep) ? src_of(G, S.in0) : -1;
    if (t >= 0 && t != c.stop && G.n[t].op == VB_RELU && lowest_consumer(G, active, t, c.start) &&
        G.n[G.n[t].in0].cons.size() == 1) {
      int z = G.n[t].in0;
      int b = B.alloc();
      const float* bias_z = nullptr;
      s = effective_bias(B, G, z, bias_z);
      if (s) return s;
      const long long off = chunk_off(z);
      HIPCHK(launch_identity_linear(S.W, (int)S.size, (int)G.n[z].size, S.b, B.lo[z] + off, B.hi[z] + off, bias_z,
                                    G.n[z].c, c.cb, B.pool[b], B.rowacc, B.st, c.sel, c.cnt, c.U));
      lam[z] = b;
      from = z;
    } else if (c.sel) {
      // selected rows are written out (2U per input) with their bias terms
      const int b = B.alloc();
      if (b < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", c.start);
      HIPCHK(launch_select_fill(c.cb, (int)S.size, c.U, c.sel, c.cnt, bias, S.c, B.pool[b], B.rowacc, B.st));
      lam[c.start] = b;
    } else {
      HIPCHK(launch_identity_bias(c.cb, (int)S.size, bias, S.c, B.rowacc, B.st));
      lam[c.start] = IDENT;
    }
  }

  for (int k = from; k > c.stop; --k) {
    if (lam[k] == -1) continue;
    const NodeInfo& nd = G.n[k];
    // implicit identity rows feed the footprint kernels of ADD / Conv nodes, unless
    // alpha slopes or kept Psi need the GEMM epilogues: then they are written out
    const bool fused = !B.alpha && !B.psi_keep;
    const bool ident = lam[k] == IDENT && fused;
    if (lam[k] == IDENT && (!fused || (nd.op != VB_ADD && nd.op != VB_CONV2D))) {
      vb_status s = materialise(k);
      if (s) return s;
    }
    const int cur = lam[k];
    if (nd.op == VB_LINEAR || nd.op == VB_CONV2D) {
      const int t = src_of(G, nd.in0);
      const NodeInfo& tn = G.n[t];
      const bool lowest = lowest_consumer(G, active, t, k);
      const int pend = lam[t];
      if (pend == IDENT) {
        vb_status s = materialise(t);
        if (s) return s;
      }
      const int pbuf = lam[t];
      int epi;
      int z = -1;
      if (t == c.stop)
        epi = (lowest && !B.a_out) ? E_CONCRETIZE : E_STORE;
      else if (tn.op == VB_RELU && lowest) {
        epi = E_RELAX;
        z = tn.in0;
        if (G.n[z].cons.size() != 1)
          return fail(VB_EUNSUPPORTED, "node %d feeds more than its ReLU; cannot relax", z);
      } else
        epi = E_STORE;
      int outb = -1;
      if (epi == E_RELAX || epi == E_STORE) {
        if (epi == E_STORE && pbuf >= 0 && B.refs[pbuf] == 1)
          outb = pbuf;  // accumulate in place
        else
          outb = B.alloc();
        if (outb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
      }
      const float* bias = nullptr;
      if (epi == E_RELAX) {
        vb_status s = effective_bias(B, G, z, bias);
        if (s) return s;
      } else if (epi == E_STORE && t != c.stop && (tn.op == VB_LINEAR || tn.op == VB_CONV2D || tn.op == VB_ADD)) {
        // (the domain node's own bias is not part of beta: the domain box is its output)
        vb_status s = effective_bias(B, G, t, bias);
        if (s) return s;
      }
      const int tgt_bounds = (epi == E_RELAX) ? z : t;
      bool direct = false;
      if (!ident && nd.op == VB_CONV2D && epi == E_CONCRETIZE) {
        vb_status s = direct_conv_input(B, nd, tn, t, rows, cur, pbuf, c, direct);
        if (s) return s;
      }
      if (ident) {
        // rows +-I over this conv's output: footprint kernel, no GEMM
        IdConv a{};
        a.W = nd.W;
        a.Co = nd.c;
        a.Ho = nd.h;
        a.Wo = nd.w;
        a.Ci = tn.c;
        a.Hi = tn.h;
        a.Wi = tn.w;
        a.kh = nd.kh;
        a.kw = nd.kw;
        a.stride = nd.stride;
        a.pad = nd.pad;
        a.mode = epi;
        a.addend = pbuf >= 0 ? B.pool[pbuf] : nullptr;
        a.out = outb >= 0 ? B.pool[outb] : nullptr;
        a.bias = bias;
        if (epi == E_RELAX) {
          a.lo = B.lo[z] + chunk_off(z);
          a.hi = B.hi[z] + chunk_off(z);
        } else if (epi == E_CONCRETIZE) {
          if (t == 0) {
            a.center = B.dom.xc + chunk_off(0);
            a.radius = B.dom.xr ? B.dom.xr + chunk_off(0) : nullptr;
            a.eps = B.dom.eps;
          } else {
            a.lo = B.lo[t] + chunk_off(t);
            a.hi = B.hi[t] + chunk_off(t);
          }
        }
        if ((long long)2 * nd.size != R) return fail(VB_ESHAPE, "internal: identity rows do not match node %d", k);
        HIPCHK(launch_identity_conv(a, c.cb, B.rowacc, B.st));
      } else if (direct) {
        // few-channel domain: the transposed conv and the concretisation in one pass
        B.release(cur);
      } else if (nd.op == VB_CONV2D && tn.c <= 8 && nd.kh * nd.kw * tn.c <= 64 && epi != E_STORE &&
                 (size_t)rows * nd.h * nd.w * nd.kh * nd.kw * tn.c <= B.pool_floats &&
                 (B.alpha == nullptr || B.alpha[t] == nullptr)) {
        // few input channels: Q = Lambda . W over (tap, c_in) columns as a dense GEMM,
        // then sum the taps per input pixel with the epilogue (no 3-of-32-column tiles)
        const int qb = B.alloc();
        if (qb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
        GemmDesc d = base_desc();
        d.M = rows * nd.h * nd.w;
        d.K = nd.c;
        d.N = nd.kh * nd.kw * tn.c;
        d.cs = d.K;
        d.a_row_stride = d.K;
        d.A = B.pool[cur];
        d.B = B.wt[k];
        d.epi = E_STORE;
        d.out = B.pool[qb];
        // algorithmic work of this layer: the forward multiply-adds per row
        const double macs = (double)rows * nd.c * tn.c * nd.kh * nd.kw * nd.h * nd.w;
        vb_status s = run_gemm_reduce(B, d, rows, 1, false, 2.0 * macs);
        if (s) return s;
        Col2Im a{};
        a.Q = B.pool[qb];
        a.Ho = nd.h;
        a.Wo = nd.w;
        a.Ci = tn.c;
        a.Hi = tn.h;
        a.Wi = tn.w;
        a.kh = nd.kh;
        a.kw = nd.kw;
        a.stride = nd.stride;
        a.pad = nd.pad;
        a.rows_per_b = (int)R;
        a.mode = epi;
        a.addend = pbuf >= 0 ? B.pool[pbuf] : nullptr;
        a.out = outb >= 0 ? B.pool[outb] : nullptr;
        a.psi_out = psi_of(t);
        a.bias = bias;
        if (epi == E_RELAX) {
          a.lo = B.lo[z] + chunk_off(z);
          a.hi = B.hi[z] + chunk_off(z);
        } else if (t == 0) {
          a.center = B.dom.xc + chunk_off(0);
          a.radius = B.dom.xr ? B.dom.xr + chunk_off(0) : nullptr;
          a.eps = B.dom.eps;
        } else {
          a.center = B.box_c;
          a.radius = B.box_r;
        }
        HIPCHK(launch_col2im(a, rows, B.rowacc, B.st));
        B.release(qb);
        B.release(cur);
      } else {
        // one launch (dense) or one per output-parity class (conv)
        std::vector<GemmDesc> descs;
        if (nd.op == VB_LINEAR) {
          descs.push_back(linear_backward(nd, tn, B.pool[cur], rows));
        } else {
          for (int py = 0; py < nd.stride; ++py)
            for (int px = 0; px < nd.stride; ++px) {
              GemmDesc d;
              if (conv_backward(nd, tn, B.pool[cur], rows, py, px, d)) descs.push_back(d);
            }
        }
        if (epi == E_RELAX)
          HIPCHK(launch_relax_coef(B.lo[z] + chunk_off(z), B.hi[z] + chunk_off(z), (long long)c.cb * G.n[z].size,
                                   aidx_of(t), B.coef, B.st));
        // output-parity classes that no tap reaches (a 1x1 stride-2 conv) contribute
        // nothing: with no bias term their positions keep the pending Lambda, or zero
        bool zero_first = false;
        for (const GemmDesc& d : descs)
          if (d.K == 0 && epi == E_STORE && bias == nullptr && pbuf < 0) zero_first = true;
        if (zero_first) HIPCHK(launch_fill(B.pool[outb], 0.f, (long long)rows * tn.size, B.st));
        bool joint = descs.size() > 1;  // the parity classes as one grid, if they share a tile shape
        for (GemmDesc& d : descs) {
          if (d.K == 0 && epi == E_STORE && bias == nullptr && (pbuf < 0 || pbuf == outb)) joint = false;
          d.B = B.wt[k];
          d.coef = B.coef;
          d.epi = epi;
          d.rows_per_b = (int)R;
          d.addend = (pbuf >= 0) ? B.pool[pbuf] : nullptr;
          d.bias = bias;
          // a Lambda over a flattened [h][w][c] node indexes its per-channel bias by n % c
          d.bias_c = G.n[tgt_bounds].c;
          if (epi != E_CONCRETIZE) d.out = B.pool[outb];
          if (epi == E_RELAX) {
            d.lo = B.lo[tgt_bounds] + chunk_off(tgt_bounds);
            d.hi = B.hi[tgt_bounds] + chunk_off(tgt_bounds);
            d.alpha = alpha_of(t);
            d.psi_out = psi_of(t);
            d.aidx = aidx_of(t);
            d.acols = acols_of(t);
          }
          if (epi == E_CONCRETIZE) {
            d.psi_out = psi_of(t);
            if (t == 0) {
              d.center = B.dom.xc + chunk_off(0);
              d.radius = B.dom.xr ? B.dom.xr + chunk_off(0) : nullptr;
              d.eps = B.dom.eps;
            } else {
              d.center = B.box_c;  // centre / radius of the domain box, this chunk
              d.radius = B.box_r;
            }
          }
        }
        const bool reduce = (epi != E_STORE) || bias != nullptr;
        // algorithmic multiply-adds of this layer for these rows (conv: the
        // forward count C_out*C_in*kh*kw*H_out*W_out per row)
        const double macs = (nd.op == VB_LINEAR) ? (double)rows * nd.size * tn.size
                                                 : (double)rows * nd.c * tn.c * nd.kh * nd.kw * nd.h * nd.w;
        vb_status s = VB_OK;
        if (joint) s = run_gemm_multi_reduce(B, descs, rows, reduce, 2.0 * macs, joint);
        if (s) return s;
        if (!joint) {
          for (GemmDesc& d : descs) {
            if (d.K == 0 && epi == E_STORE && bias == nullptr && (pbuf < 0 || pbuf == outb)) continue;
            // (the multiply-adds split evenly over the output-parity launches)
            s = run_gemm_reduce(B, d, rows, d.gh * d.gw, reduce, 2.0 * macs / descs.size());
            if (s) return s;
          }
        }
        if (epi == E_RELAX && B.beta && B.beta->split && B.beta->split[t] && B.beta->beta && B.beta->beta[t]) {
          // split constraints at this ReLU: Lambda over z -= beta * split (and its bias terms)
          const long long nz = G.n[z].size;
          HIPCHK(launch_beta_apply(B.pool[outb], rows, (int)R, (int)nz, B.beta->beta[t] + (long long)c.b0 * R * nz,
                                   B.beta->split[t] + (long long)c.b0 * nz, bias, G.n[z].c, B.rowacc, B.st));
        }
        B.release(cur);
      }
      lam[k] = -1;
      if (epi == E_RELAX) {
        if (pbuf >= 0) {
          B.release(pbuf);
          lam[t] = -1;
        }
        lam[z] = outb;
      } else if (epi == E_CONCRETIZE) {
        if (pbuf >= 0) {
          B.release(pbuf);
          lam[t] = -1;
        }
      } else {
        if (pbuf >= 0 && outb != pbuf) B.release(pbuf);
        lam[t] = outb;
      }
    } else if (nd.op == VB_RELU) {
      // Lambda accumulated without a fused consumer: standalone relaxation
      const int z = nd.in0;
      if (G.n[z].cons.size() != 1) return fail(VB_EUNSUPPORTED, "node %d feeds more than its ReLU", z);
      int outb = B.alloc();
      if (outb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
      const float* bias_z = nullptr;
      vb_status s = effective_bias(B, G, z, bias_z);
      if (s) return s;
      const int P = nd.h * nd.w;
      HIPCHK(launch_relax(B.pool[cur], 0, 1.f, nullptr, rows, (int)R, P, nd.c, B.lo[z] + chunk_off(z),
                          B.hi[z] + chunk_off(z), bias_z, alpha_of(k), psi_of(k), aidx_of(k), acols_of(k),
                          B.pool[outb], B.rowacc, B.st));
      B.release(cur);
      lam[k] = -1;
      if (lam[z] != -1) return fail(VB_EUNSUPPORTED, "internal: node %d already has a pending Lambda", z);
      lam[z] = outb;
    } else if (nd.op == VB_ADD) {
      const int ins[2] = {nd.in0, nd.in1};
      const int nin = nd.in0 == nd.in1 ? 1 : 2;
      for (int q = 0; q < nin; ++q) {
        const int t = ins[q];
        if (nin == 1) {
          // x + x: Lambda flows twice into x
          int b = B.alloc();
          if (b < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
          HIPCHK(launch_add(B.pool[cur], B.pool[cur], 1.f, B.pool[b], (long long)rows * G.n[t].size, B.st));
          vb_status s = accumulate(t, b);
          if (s) return s;
        } else if (cur == IDENT) {
          if (lam[t] == -1) {
            lam[t] = IDENT;
          } else {
            int b = B.alloc();
            if (b < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
            HIPCHK(launch_identity_fill(c.cb, (int)S.size, B.pool[b], B.st));
            vb_status s = accumulate(t, b);
            if (s) return s;
          }
        } else {
          B.refs[cur]++;
          vb_status s = accumulate(t, cur);
          if (s) return s;
        }
      }
      if (cur >= 0) B.release(cur);
      lam[k] = -1;
    } else if (nd.op == VB_GAP) {
      const int t = nd.in0;
      const NodeInfo& tn = G.n[t];
      const int P = tn.h * tn.w;
      const float scale = 1.f / (float)P;
      if (lam[t] == IDENT) {
        vb_status s = materialise(t);
        if (s) return s;
      }
      const int pend = lam[t];
      if (tn.op == VB_RELU && lowest_consumer(G, active, t, k) && t != c.stop) {
        const int z = tn.in0;
        if (G.n[z].cons.size() != 1) return fail(VB_EUNSUPPORTED, "node %d feeds more than its ReLU", z);
        int outb = B.alloc();
        if (outb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
        const float* bias_z = nullptr;
        vb_status s = effective_bias(B, G, z, bias_z);
        if (s) return s;
        HIPCHK(launch_relax(B.pool[cur], 1, scale, pend >= 0 ? B.pool[pend] : nullptr, rows, (int)R, P, tn.c,
                            B.lo[z] + chunk_off(z), B.hi[z] + chunk_off(z), bias_z, alpha_of(t), psi_of(t),
                            aidx_of(t), acols_of(t), B.pool[outb], B.rowacc, B.st));
        if (pend >= 0) {
          B.release(pend);
          lam[t] = -1;
        }
        lam[z] = outb;
      } else {
        int outb = (pend >= 0 && B.refs[pend] == 1) ? pend : B.alloc();
        if (outb < 0) return fail(VB_EUNSUPPORTED, "internal: lambda pool exhausted at node %d", k);
        HIPCHK(launch_gap_expand(B.pool[cur], rows, P, tn.c, scale, pend >= 0 ? B.pool[pend] : nullptr,
                                 B.pool[outb], B.st));
        if (pend >= 0 && pend != outb) B.release(pend);
        lam[t] = outb;
      }
      B.release(cur);
      lam[k] = -1;
    } else if (nd.op == VB_FLATTEN) {
      vb_status s = accumulate(nd.in0, cur);
      if (s) return s;
      lam[k] = -1;
    } else {
      return fail(VB_EUNSUPPORTED, "cannot back-substitute through node %d (op %d)", k, nd.op);
    }
  }
  if (lam[c.stop] == IDENT) {
    vb_status s = materialise(c.stop);
    if (s) return s;
  }
  if (B.a_out) {
    // Lambda over the domain node and beta (rowacc before concretisation)
    const long long sz = G.n[c.stop].size;
    float* dst = B.a_out + (long long)c.b0 * R * sz;
    if (lam[c.stop] >= 0)
      HIPCHK(hipMemcpyAsync(dst, B.pool[lam[c.stop]], (size_t)rows * sz * sizeof(float), hipMemcpyDeviceToDevice,
                            B.st));
    else
      HIPCHK(launch_fill(dst, 0.f, (long long)rows * sz, B.st));
    if (B.bias_out)
      HIPCHK(hipMemcpyAsync(B.bias_out + (long long)c.b0 * R, B.rowacc, (size_t)rows * sizeof(float),
                            hipMemcpyDeviceToDevice, B.st));
  }
  if (lam[c.stop] >= 0) {
    const NodeInfo& sn = G.n[c.stop];
    const long long off = (long long)c.b0 * sn.size;
    if (c.stop == 0)
      HIPCHK(launch_concretize_rows(B.pool[lam[c.stop]], rows, (int)sn.size, (int)R, B.dom.xc + off,
                                    B.dom.xr ? B.dom.xr + off : nullptr, B.dom.eps, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, B.rowacc, B.st));
    else
      HIPCHK(launch_concretize_rows(B.pool[lam[c.stop]], rows, (int)sn.size, (int)R, nullptr, nullptr, 0.f,
                                    B.lo[c.stop] + off, B.hi[c.stop] + off, nullptr, nullptr, nullptr, B.rowacc,
                                    B.st));
  }
  return VB_OK;
}

// Widest Lambda and largest partial buffer of a back-substitution, per batch element.
void bwd_requirements(const Graph& G, int start, int stop, long long R, long long& maxw, long long& part_per_b) {
  maxw = 0;
  part_per_b = 0;
  std::vector<char> active(G.n.size(), 0);
  std::vector<int> stack{start};
  while (!stack.empty()) {
    int k = stack.back();
    stack.pop_back();
    if (active[k] || k < stop) continue;
    active[k] = 1;
    if (k == stop || k == 0) continue;
    stack.push_back(G.n[k].in0);
    if (G.n[k].op == VB_ADD) stack.push_back(G.n[k].in1);
  }
  for (size_t k = 0; k < G.n.size(); ++k) {
    if (!active[k]) continue;
    const NodeInfo& nd = G.n[k];
    maxw = std::max(maxw, nd.size);
    if ((nd.op == VB_LINEAR || nd.op == VB_CONV2D) && (int)k != stop) {
      const NodeInfo& in = G.n[src_of(G, nd.in0)];
      const long long n_ch = (nd.op == VB_LINEAR) ? in.size : in.c;
      const int bn = n_ch > 64 ? 128 : (n_ch > 32 ? 64 : 32);
      const long long S = (n_ch + bn - 1) / bn;
      const long long P = (nd.op == VB_LINEAR) ? 1 : (long long)in.h * in.w;
      part_per_b = std::max(part_per_b, R * P * S);
    }
  }
}

// Floats of the transposed weight copies (and summed ADD biases) at the head
// of the workspace.
size_t wt_floats(const Graph& G) {
  size_t f = 0;
  for (const NodeInfo& n : G.n) {
    if (n.op == VB_LINEAR) f += align_up((size_t)n.size * G.n[n.in0].size * 4) / 4;
    if (n.op == VB_CONV2D) f += align_up((size_t)n.kh * n.kw * n.c * G.n[n.in0].c * 4) / 4;
    if (n.op == VB_ADD) f += align_up((size_t)n.c * 4) / 4;
  }
  return f;
}

// Write W^T of every affine node into ws (Linear: [n_in][n_out]; Conv: per tap
// [c_in][c_out]) and the per-node bias a Lambda carries into beta (for an ADD:
// the sum of its inputs' biases); return the per-node pointers.
// Transposed weights and summed ADD biases at the head of the workspace, and
// their addresses; with launch false only the addresses (the copies are
// already there from an earlier call on the same workspace).
vb_status prepare_weights(const Graph& G, char* ws, hipStream_t st, std::vector<const float*>& wt,
                          std::vector<const float*>& beff, bool launch = true) {
  wt.assign(G.n.size(), nullptr);
  beff.assign(G.n.size(), nullptr);
  float* p = (float*)ws;
  for (size_t k = 0; k < G.n.size(); ++k) {
    const NodeInfo& n = G.n[k];
    if (n.op == VB_LINEAR) {
      const int nin = (int)G.n[n.in0].size;
      if (launch) HIPCHK(launch_transpose(n.W, 1, (int)n.size, nin, p, st));
      wt[k] = p;
      beff[k] = n.b;
      p += align_up((size_t)n.size * nin * 4) / 4;
    } else if (n.op == VB_CONV2D) {
      const int cin = G.n[n.in0].c;
      if (launch) HIPCHK(launch_transpose(n.W, n.kh * n.kw, n.c, cin, p, st));
      wt[k] = p;
      beff[k] = n.b;
      p += align_up((size_t)n.kh * n.kw * n.c * cin * 4) / 4;
    } else if (n.op == VB_ADD) {
      std::vector<const float*> terms;
      bias_terms(G, (int)k, terms);
      if (terms.size() == 1) {
        beff[k] = terms[0];
      } else if (terms.size() > 1) {
        if (launch) {
          HIPCHK(launch_add(terms[0], terms[1], 1.f, p, n.c, st));
          for (size_t i = 2; i < terms.size(); ++i) HIPCHK(launch_add(p, terms[i], 1.f, p, n.c, st));
        }
        beff[k] = p;
      }
      p += align_up((size_t)n.c * 4) / 4;
    }
  }
  return VB_OK;
}

struct WsLayout {
  size_t pool_floats;  // per buffer
  size_t part_floats;
  size_t rows;
  size_t box_floats;   // centre and radius of a box domain, each
  size_t coef_floats;  // relaxation coefficients (float4 per neuron of one batch chunk)
  size_t bytes;
};

// The largest node between the domain node (exclusive) and the start node.
long long region_max_size(const Graph& G, int start, int stop) {
  long long m = 0;
  for (int k = stop + 1; k <= start; ++k) m = std::max(m, G.n[k].size);
  return m;
}

// coef_per_b: neurons per batch element of the largest node whose relaxation
// coefficients a back-substitution builds (0: maxw, the widest Lambda row,
// which covers it when Lambda rows are as wide as the nodes).
WsLayout layout_for(long long maxw, long long part_per_b, long long R, int cb, size_t extra_floats,
                    long long box_per_b = 0, long long coef_per_b = 0) {
  WsLayout L;
  L.pool_floats = (size_t)cb * R * maxw;
  L.part_floats = (size_t)cb * part_per_b;
  L.rows = (size_t)cb * R;
  L.box_floats = (size_t)cb * box_per_b;
  L.coef_floats = 4 * (size_t)cb * std::max(maxw, coef_per_b);
  L.bytes = NPOOL * align_up(L.pool_floats * 4) + align_up(L.part_floats * 4) + align_up(L.rows * 4) +
            2 * align_up(L.box_floats * 4) + align_up(L.coef_floats * 4) + align_up(extra_floats * 4);
  return L;
}

// Run a back-substitution over the whole batch in chunks that fit `ws`.
// For each chunk, `after` is called with (rowacc, b0, cb) to consume the row bounds.
// How a back-substitution of R rows per batch element from `start` to `stop`
// is chunked over the batch: the largest chunk whose workspace fits ws_bytes
// (and whose GEMM index spaces stay 32-bit).  `plain` rows (identity rows
// without returned linear bounds, alpha or kept Psi) may take the footprint
// path; `spec` rows widen Lambda to the start node.
struct ChunkPlan {
  int cb;
  WsLayout L;
};

vb_status plan_chunks(const Graph& G, int start, int stop, long long R, bool plain, bool spec, int batch,
                      size_t ws_bytes, size_t reserved_floats, ChunkPlan& plan) {
  long long maxw, ppb;
  if (!plain || (!patch_requirements(G, start, stop, R, maxw, ppb) && !window_requirements(G, start, stop, R, maxw, ppb)))
    bwd_requirements(G, start, stop, R, maxw, ppb);
  if (spec) maxw = std::max(maxw, G.n[start].size);
  const long long box = stop > 0 ? G.n[stop].size : 0;
  // GEMM index spaces are 32-bit: rows x pixels (padded to whole row blocks) per launch
  long long maxp = 1;
  for (size_t k = 1; k < G.n.size(); ++k) {
    const NodeInfo& nd = G.n[k];
    if (nd.op != VB_CONV2D || (int)k > start || (int)k <= stop) continue;
    const NodeInfo& in = G.n[src_of(G, nd.in0)];
    maxp = std::max(maxp, std::max((long long)in.h * in.w, (long long)nd.h * nd.w));
  }
  auto fits_index = [&](long long cbn) { return cbn * R * maxp + 64 * maxp + 256 <= (long long)INT32_MAX; };
  int cb = batch;
  // footprint rows keep Lambda on windows narrower than the nodes, but the
  // relaxation coefficients cover whole nodes
  const long long coef = region_max_size(G, start, stop);
  while (cb > 1 && (!fits_index(cb) || layout_for(maxw, ppb, R, cb, reserved_floats, box, coef).bytes > ws_bytes))
    cb = (cb + 1) / 2;
  if (!fits_index(cb))
    return fail(VB_EUNSUPPORTED, "one batch element has %lld rows x %lld pixels: beyond the 32-bit GEMM index range",
                R, maxp);
  plan.cb = cb;
  plan.L = layout_for(maxw, ppb, R, cb, reserved_floats, box, coef);
  if (plan.L.bytes > ws_bytes)
    return fail(VB_ENOMEM, "workspace of %zu bytes is too small: one batch element needs %zu", ws_bytes, plan.L.bytes);
  return VB_OK;
}

// Run a back-substitution over the whole batch in chunks that fit `ws`.
// For each chunk, `after` is called with (rowacc, b0, cb) to consume the row bounds.
template <class After>
vb_status backward_all(Backward& B, int start, int stop, const float* C, int m, int split, int batch, long long R,
                       char* ws, size_t ws_bytes, size_t reserved_floats, After after) {
  ChunkPlan plan;
  const bool plain = !(C || B.a_out || B.alpha || B.psi_keep);
  vb_status s0 = plan_chunks(B.G, start, stop, R, plain, C != nullptr, batch, ws_bytes, reserved_floats, plan);
  if (s0) return s0;
  const int cb = plan.cb;
  const WsLayout& L = plan.L;
  char* p = ws + align_up(reserved_floats * 4);
  for (int i = 0; i < NPOOL; ++i) {
    B.pool[i] = (float*)p;
    p += align_up(L.pool_floats * 4);
  }
  B.pool_floats = L.pool_floats;
  B.part = (float*)p;
  B.part_floats = L.part_floats;
  p += align_up(L.part_floats * 4);
  B.rowacc = (float*)p;
  p += align_up(L.rows * 4);
  B.box_c = (float*)p;
  p += align_up(L.box_floats * 4);
  B.box_r = (float*)p;
  p += align_up(L.box_floats * 4);
  B.coef = (float4*)p;
  for (int b0 = 0; b0 < batch; b0 += cb) {
    const int n = std::min(cb, batch - b0);
    BwdCall c;
    c.start = start;
    c.stop = stop;
    c.C = C ? C + (long long)b0 * m * B.G.n[start].size : nullptr;
    c.m = m;
    c.split = split;
    c.b0 = b0;
    c.cb = n;
    c.batch_total = batch;
    if (B.sel) {
      c.sel = B.sel + (long long)b0 * B.G.n[start].size;
      c.cnt = B.cnt + b0;
      c.U = B.U;
    }
    B.live_cnt = c.cnt;
    B.live_u = c.U;
    vb_status s = backward_chunk(B, c, R);
    B.live_cnt = nullptr;
    if (s) return s;
    s = after(B.rowacc, b0, n);
    if (s) return s;
  }
  return VB_OK;
}

bool one_affine_step(const Graph& G, int z, int stop) {
  const NodeInfo& n = G.n[z];
  if (n.op != VB_LINEAR && n.op != VB_CONV2D) return false;
  return src_of(G, n.in0) == stop;
}

// ---------------------------------------------------------------------------
// IBP

// Split-K factor of the IBP GEMM of an affine node (small grids split K over
// more workgroups) and the workspace its partial sums take.
int ibp_gemm_split(const GemmDesc& d) {
  const long long tiles = (long long)((d.M + 127) / 128) * ((d.N + 127) / 128);
  const int stages = (d.K + 31) / 32;
  int S = 1;
  while (tiles * S * 2 <= 512 && stages / (S * 2) >= 4) S *= 2;
  return S;
}

// Workspace that lets every affine node's IBP take its split-K path.
size_t ibp_workspace(const Graph& G, int batch) {
  size_t best = 0;
  for (size_t k = 1; k < G.n.size(); ++k) {
    const NodeInfo& nd = G.n[k];
    if (nd.op != VB_LINEAR && nd.op != VB_CONV2D) continue;
    const NodeInfo& in = G.n[src_of(G, nd.in0)];
    size_t need;
    if (nd.op == VB_LINEAR && batch <= 16 && in.size % 4 == 0) {
      need = 2ull * ibp_narrow_slices(nd.c, (int)in.size) * batch * nd.c * sizeof(float);
    } else {
      const GemmDesc d = affine_forward(nd, in, batch);
      need = 2ull * ibp_gemm_split(d) * d.M * d.N * sizeof(float);
    }
    best = std::max(best, need);
  }
  return best;
}

// Which nodes IBP writes, checked before anything is launched: a node is
// skipped when its bounds storage is NULL, which is an error if another node
// reads its bounds (affine nodes read their source through flatten nodes; the
// spec fold reads the last node's source).  Patterns the kernels do not take
// (ReLU / ADD / GAP / FLATTEN fed by the input node) are rejected here too.
vb_status ibp_plan(const Graph& G, float* const* lo, float* const* hi, bool spec, std::vector<char>& skip) {
  const int N = (int)G.n.size();
  skip.assign(N, 0);
  std::vector<char> needed(N, 0);
  for (int k = 1; k < N; ++k) {
    const NodeInfo& nd = G.n[k];
    switch (nd.op) {
      case VB_LINEAR:
      case VB_CONV2D:
        needed[src_of(G, nd.in0)] = 1;
        break;
      case VB_RELU:
      case VB_GAP:
      case VB_FLATTEN:
        if (nd.in0 == 0) return fail(VB_EUNSUPPORTED, "node %d: op %d directly on the input node", k, nd.op);
        needed[nd.in0] = 1;
        break;
      case VB_ADD:
        if (nd.in0 == 0 || nd.in1 == 0) return fail(VB_EUNSUPPORTED, "node %d: ADD directly on the input node", k);
        needed[nd.in0] = needed[nd.in1] = 1;
        break;
      default:
        return fail(VB_EUNSUPPORTED, "IBP through node %d (op %d)", k, nd.op);
    }
  }
  if (spec) needed[src_of(G, G.n[G.L].in0)] = 1;
  for (int k = 1; k < N; ++k) {
    const bool has = lo[k] && hi[k];
    if (!has && needed[k]) return fail(VB_EINVAL, "node %d: IBP needs node_lo/node_hi storage (its bounds are read)", k);
    if ((lo[k] == nullptr) != (hi[k] == nullptr)) return fail(VB_EINVAL, "node %d: only one of node_lo/node_hi given", k);
    skip[k] = !has;
  }
  return VB_OK;
}

vb_status ibp_impl(const Graph& G, int batch, const float* xc, const float* xr, float eps, float* const* lo,
                   float* const* hi, hipStream_t st, void* ws = nullptr, size_t ws_bytes = 0, bool spec = false) {
  const int N = (int)G.n.size();
  std::vector<char> done;
  vb_status s0 = ibp_plan(G, lo, hi, spec, done);
  if (s0) return s0;
  for (int k = 1; k < N; ++k) {
    const NodeInfo& nd = G.n[k];
    if (done[k]) continue;
    const int p = nd.in0;
    const int ps = src_of(G, p);
    switch (nd.op) {
      case VB_LINEAR:
      case VB_CONV2D: {
        const float* a1 = ps == 0 ? xc : lo[ps];
        const float* a2 = ps == 0 ? xr : hi[ps];
        if (nd.op == VB_LINEAR && ibp_narrow_fits(batch, (int)G.n[ps].size, nd.W, a1, a2)) {
          // small batch: stream the weights once (batch on the MFMA columns)
          NarrowIbp q{};
          q.batch = batch;
          q.K = (int)G.n[ps].size;
          q.N = nd.c;
          q.amode = ps == 0 ? A_IBP_BALL : A_IBP_BOX;
          q.A = a1;
          q.A2 = a2;
          q.eps = eps;
          q.W = nd.W;
          if (nd.Wp && q.K % 16 == 0) {
            q.W = nd.Wp;
            q.packed = 1;
          }
          q.bias = nd.b;
          q.lo = lo[k];
          q.hi = hi[k];
          if (nd.cons.size() == 1 && G.n[nd.cons[0]].op == VB_RELU && lo[nd.cons[0]] && hi[nd.cons[0]]) {
            q.relu_lo = lo[nd.cons[0]];
            q.relu_hi = hi[nd.cons[0]];
            done[nd.cons[0]] = 1;
          }
          int S = ibp_narrow_slices(q.N, q.K);
          const size_t need = 2ull * S * batch * q.N * sizeof(float);
          if (S > 1 && (!ws || need > ws_bytes)) S = 1;
          if (S > 1) {
            q.pc = (float*)ws;
            q.pr = q.pc + (size_t)S * batch * q.N;
          }
          HIPCHK(launch_ibp_narrow(q, S, st));
          break;
        }
        GemmDesc d = affine_forward(nd, G.n[ps], batch);
        d.epi = E_IBP;
        if (ps == 0) {
          d.amode = A_IBP_BALL;
          d.A = xc;
          d.A2 = xr;
          d.eps = eps;
        } else {
          d.amode = A_IBP_BOX;
          d.A = lo[ps];
          d.A2 = hi[ps];
        }
        d.out = lo[k];
        d.out2 = hi[k];
        d.bias = nd.b;
        if (nd.cons.size() == 1 && G.n[nd.cons[0]].op == VB_RELU && lo[nd.cons[0]] && hi[nd.cons[0]]) {
          d.relu_lo = lo[nd.cons[0]];
          d.relu_hi = hi[nd.cons[0]];
          done[nd.cons[0]] = 1;
        }
        // small grids (a Linear over a small batch): split K over more workgroups
        const int S = ibp_gemm_split(d);
        const size_t need = 2ull * S * d.M * d.N * sizeof(float);
        if (S > 1 && ws && need <= ws_bytes) {
          float* pc = (float*)ws;
          float* pr = pc + (size_t)S * d.M * d.N;
          GemmDesc e = d;
          e.ksplit = S;
          e.out = pc;
          e.out2 = pr;
          HIPCHK(launch_gemm(e, st));
          HIPCHK(launch_ibp_splitk_finish(pc, pr, S, (long long)d.M * d.N, d.N, nd.b, lo[k], hi[k], d.relu_lo,
                                          d.relu_hi, st));
        } else {
          HIPCHK(launch_gemm(d, st));
        }
        break;
      }
      case VB_RELU:
        HIPCHK(launch_ibp_eltwise(0, lo[p], hi[p], nullptr, nullptr, lo[k], hi[k], (long long)batch * nd.size, st));
        break;
      case VB_ADD:
        HIPCHK(launch_ibp_eltwise(1, lo[nd.in0], hi[nd.in0], lo[nd.in1], hi[nd.in1], lo[k], hi[k],
                                  (long long)batch * nd.size, st));
        break;
      case VB_GAP:
        HIPCHK(launch_ibp_gap(lo[p], hi[p], batch, G.n[p].h * G.n[p].w, G.n[p].c, lo[k], hi[k], st));
        break;
      case VB_FLATTEN:
        if (lo[k] != lo[p]) HIPCHK(launch_add(lo[p], nullptr, 0.f, lo[k], (long long)batch * nd.size, st));
        if (hi[k] != hi[p]) HIPCHK(launch_add(hi[p], nullptr, 0.f, hi[k], (long long)batch * nd.size, st));
        break;
      default:
        return fail(VB_EUNSUPPORTED, "IBP through node %d (op %d)", k, nd.op);
    }
  }
  return VB_OK;
}

vb_status check_domain(const float* xc) {
  if (!xc) return fail(VB_EINVAL, "x_center is NULL");
  return VB_OK;
}

}  // namespace

// ===========================================================================
// C ABI

extern "C" const char* vb_last_error(void) { return g_err.c_str(); }

// Ints kept after the weight copies by unstable-only rows: per input a neuron
// ranking and a neuron list over the widest node, and a count.
static size_t select_floats(const Graph& G, int batch) {
  long long n = 0;
  for (const NodeInfo& nd : G.n) n = std::max(n, nd.size);
  return 2 * (align_up((size_t)batch * n * 4) / 4) + align_up((size_t)batch * 4) / 4;
}

static size_t crown_workspace(const Graph& G, int batch, int m, int method, int region_start,
                              bool unstable_only = false) {
  size_t best = 0;
  const size_t reserved = wt_floats(G) + (unstable_only ? select_floats(G, batch) : 0);
  auto consider = [&](int start, int stop, long long R, bool spec) {
    long long maxw, ppb;
    if (spec || (!patch_requirements(G, start, stop, R, maxw, ppb) && !window_requirements(G, start, stop, R, maxw, ppb)))
      bwd_requirements(G, start, stop, R, maxw, ppb);
    if (spec) maxw = std::max(maxw, G.n[start].size);
    best = std::max(best, layout_for(maxw, ppb, R, batch, reserved, stop > 0 ? G.n[stop].size : 0,
                                     region_max_size(G, start, stop)).bytes);
  };
  const int L = G.L;
  if (m > 0) {
    consider(L, src_of(G, G.n[L].in0), 2LL * m, true);  // IBP spec fold
    consider(L, 0, 2LL * m, true);
  }
  if (method != VB_METHOD_IBP) {
    const int stop = method == VB_METHOD_CROWN ? 0 : region_start;
    for (size_t r = 0; r < G.n.size(); ++r) {
      if (G.n[r].op != VB_RELU) continue;
      int z = G.n[r].in0;
      if (z <= stop || one_affine_step(G, z, stop)) continue;
      consider(z, stop, 2LL * G.n[z].size, false);
    }
    if (m > 0 && method == VB_METHOD_HYBRID) consider(L, stop, 2LL * m, true);
  }
  return best;
}

namespace {
bool alpha_chain(const Graph& G, std::vector<std::pair<int, int>>& chain);
size_t alpha_workspace(const Graph& G, int batch, int m, const int* width = nullptr);
size_t alpha_workspace_at(const Graph& G, int batch, int start, long long R, bool spec, const int* width,
                          bool with_beta = false);
vb_status check_compact(const Graph& G, int batch, int m, const vb_alpha_compact* c);
}  // namespace

extern "C" vb_status vb_workspace_size(const vb_graph* g, int32_t batch, int32_t m, int32_t method,
                                       int32_t region_start, size_t* bytes) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (!bytes) return fail(VB_EINVAL, "bytes is NULL");
  if (batch <= 0 || m < 0) return fail(VB_EINVAL, "batch must be > 0 and m >= 0");
  const bool alpha_rows = (method & VB_ALPHA_ROWS) != 0;
  const bool unstable_only = (method & VB_UNSTABLE_ONLY) != 0;
  method &= ~(VB_INTERSECT_IBP | VB_ALPHA_ROWS | VB_UNSTABLE_ONLY);
  if (method < VB_METHOD_IBP || method > VB_METHOD_HYBRID) return fail(VB_EINVAL, "unknown method %d", method);
  if (method == VB_METHOD_HYBRID && (region_start <= 0 || region_start >= G.L))
    return fail(VB_EINVAL, "region_start %d out of range", region_start);
  *bytes = std::max(crown_workspace(G, batch, m, method, region_start, unstable_only), ibp_workspace(G, batch));
  std::vector<std::pair<int, int>> chain;
  if (m > 0 && alpha_chain(G, chain)) *bytes = std::max(*bytes, alpha_workspace(G, batch, m));
  if (alpha_rows && alpha_chain(G, chain)) {
    // alpha steps on the identity rows of every ReLU input more than one affine step from the input
    for (size_t r = 0; r < G.n.size(); ++r) {
      if (G.n[r].op != VB_RELU) continue;
      const int z = G.n[r].in0;
      if (one_affine_step(G, z, 0)) continue;
      *bytes = std::max(*bytes, alpha_workspace_at(G, batch, z, 2LL * G.n[z].size, false, nullptr));
    }
  }
  return VB_OK;
}

static vb_status spec_ibp(const Graph& G, int batch, const float* C, int m, const float* const* lo,
                          const float* const* hi, float* spec_lo, float* spec_hi, void* ws, size_t ws_bytes,
                          hipStream_t st, bool weights_ready = false) {
  const int L = G.L;
  if (G.n[L].op != VB_LINEAR) return fail(VB_EUNSUPPORTED, "spec bounds need a LINEAR last node");
  const int stop = src_of(G, G.n[L].in0);
  if (stop == 0) return fail(VB_EUNSUPPORTED, "spec IBP over a single affine layer: use CROWN (exact)");
  Backward B{G, st, lo, hi, {nullptr, nullptr, 0.f}};
  vb_status s = prepare_weights(G, (char*)ws, st, B.wt, B.beff, !weights_ready);
  if (s) return s;
  return backward_all(B, L, stop, C, m, 1, batch, 2LL * m, (char*)ws, ws_bytes, wt_floats(G),
                      [&](float* acc, int b0, int cb) -> vb_status {
                        HIPCHK(launch_finish(acc, cb, m, spec_lo ? spec_lo + (long long)b0 * m : nullptr,
                                             spec_hi ? spec_hi + (long long)b0 * m : nullptr, nullptr, st));
                        return VB_OK;
                      });
}

extern "C" vb_status vb_pack_linear_bytes(int32_t n_out, int32_t n_in, size_t* bytes) {
  if (!bytes) return fail(VB_EINVAL, "bytes is NULL");
  if (n_out <= 0 || n_in <= 0 || n_in % 16 != 0)
    return fail(VB_EINVAL, "pack_linear: n_out > 0 and n_in a positive multiple of 16 (got %d, %d)", n_out, n_in);
  *bytes = pack_linear_floats(n_out, n_in) * sizeof(float);
  return VB_OK;
}

extern "C" vb_status vb_pack_linear(const float* weight, int32_t n_out, int32_t n_in, float* dst, size_t dst_bytes,
                                    void* stream) {
  size_t need = 0;
  if (vb_status s = vb_pack_linear_bytes(n_out, n_in, &need)) return s;
  if (!weight || !dst) return fail(VB_EINVAL, "pack_linear: weight or dst is NULL");
  if (((uintptr_t)dst & 15) != 0) return fail(VB_EINVAL, "pack_linear: dst must be 16-byte aligned");
  if (dst_bytes < need) return fail(VB_ENOMEM, "pack_linear: dst holds %zu bytes, the copy needs %zu", dst_bytes, need);
  HIPCHK(launch_pack_linear(weight, n_out, n_in, dst, (hipStream_t)stream));
  return VB_OK;
}

extern "C" vb_status vb_ibp(const vb_graph* g, int32_t batch, const float* x_center, const float* x_radius,
                            float eps, float* const* node_lo, float* const* node_hi, const float* C, int32_t m,
                            float* spec_lo, float* spec_hi, void* ws, size_t ws_bytes, void* stream) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (batch <= 0) return fail(VB_EINVAL, "batch must be positive");
  if ((s = check_domain(x_center))) return s;
  if (!node_lo || !node_hi) return fail(VB_EINVAL, "node_lo/node_hi arrays are NULL");
  if (!x_radius && !(eps >= 0.f)) return fail(VB_EINVAL, "eps must be >= 0");
  if (C && m <= 0) return fail(VB_EINVAL, "m must be positive with C");
  if (C && !ws) return fail(VB_EINVAL, "spec bounds need a workspace");
  if (C) {
    if (G.n[G.L].op != VB_LINEAR) return fail(VB_EUNSUPPORTED, "spec bounds need a LINEAR last node");
    if (src_of(G, G.n[G.L].in0) == 0)
      return fail(VB_EUNSUPPORTED, "spec IBP over a single affine layer: use CROWN (exact)");
    const size_t need = crown_workspace(G, 1, m, VB_METHOD_IBP, 0);
    if (ws_bytes < need)
      return fail(VB_ENOMEM, "workspace of %zu bytes is too small: one batch element needs %zu", ws_bytes, need);
  }
  hipStream_t st = (hipStream_t)stream;
  s = ibp_impl(G, batch, x_center, x_radius, eps, node_lo, node_hi, st, ws, ws_bytes, C != nullptr);
  if (s) return s;
  if (C) return spec_ibp(G, batch, C, m, node_lo, node_hi, spec_lo, spec_hi, ws, ws_bytes, st);
  return VB_OK;
}

// Spec rows with ub == NULL propagate only the rows C (lower bound); every
// other call propagates [rows; -rows].  alpha (per node, ReLU nodes
// [batch][m][size]) replaces the adaptive lower slope on unstable neurons.
static vb_status crown_backward_impl(const Graph& G, int batch, int start, int stop, const float* C, int m,
                                     const float* const* lo, const float* const* hi, Domain dom, float* lb,
                                     float* ub, void* ws, size_t ws_bytes, hipStream_t st, float* a_out = nullptr,
                                     float* bias_out = nullptr, const float* const* alpha = nullptr,
                                     bool intersect = false, const vb_alpha_compact* compact = nullptr,
                                     bool weights_ready = false, const int* sel = nullptr, const int* cnt = nullptr,
                                     int U = 0, size_t extra_reserved = 0) {
  Backward B{G, st, lo, hi, dom};
  B.sel = sel;
  B.cnt = cnt;
  B.U = U;
  B.a_out = a_out;
  B.bias_out = bias_out;
  B.alpha = alpha;
  if (alpha && compact) {
    B.aidx = compact->index;
    B.awidth = compact->width;
  }
  vb_status s = prepare_weights(G, (char*)ws, st, B.wt, B.beff, !weights_ready);
  if (s) return s;
  const bool lower_only = C && !ub;
  const long long R = C ? (lower_only ? m : 2LL * m) : (sel ? 2LL * U : 2LL * G.n[start].size);
  const int half = (int)(R / 2);
  const int n_start = (int)G.n[start].size;
  return backward_all(B, start, stop, C, m, lower_only ? 0 : 1, batch, R, (char*)ws, ws_bytes,
                      wt_floats(G) + extra_reserved, [&](float* acc, int b0, int cb) -> vb_status {
                        if (sel) {
                          HIPCHK(launch_finish_select(acc, cb, U, n_start, sel + (long long)b0 * n_start, cnt + b0,
                                                      lb ? lb + (long long)b0 * n_start : nullptr,
                                                      ub ? ub + (long long)b0 * n_start : nullptr, intersect ? 1 : 0,
                                                      st));
                        } else if (lower_only) {
                          HIPCHK(launch_finish_lower(acc, (long long)cb * m, lb ? lb + (long long)b0 * m : nullptr,
                                                     nullptr, 0, st));
                        } else {
                          HIPCHK(launch_finish(acc, cb, half, lb ? lb + (long long)b0 * half : nullptr,
                                               ub ? ub + (long long)b0 * half : nullptr, nullptr, st,
                                               intersect ? 1 : 0));
                        }
                        return VB_OK;
                      });
}

extern "C" vb_status vb_crown_backward(const vb_graph* g, int32_t batch, int32_t start, int32_t stop, const float* C,
                                       int32_t m, const float* const* node_lo, const float* const* node_hi,
                                       const vb_alpha_compact* compact, const float* const* alpha,
                                       const float* x_center, const float* x_radius, float eps, float* lb, float* ub,
                                       float* A_out, float* bias_out, void* ws, size_t ws_bytes, void* stream) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (batch <= 0) return fail(VB_EINVAL, "batch must be positive");
  if (start <= 0 || start >= (int)G.n.size()) return fail(VB_EINVAL, "start %d out of range", start);
  if (stop < 0 || stop >= start) return fail(VB_EINVAL, "stop %d must be in [0, start)", stop);
  if (C && m <= 0) return fail(VB_EINVAL, "m must be positive with C");
  if (!node_lo || !node_hi) return fail(VB_EINVAL, "node_lo/node_hi arrays are NULL");
  if (stop == 0 && (s = check_domain(x_center))) return s;
  if (stop == 0 && !x_radius && !(eps >= 0.f)) return fail(VB_EINVAL, "eps must be >= 0");
  if (!ws) return fail(VB_EINVAL, "workspace is NULL");
  if (bias_out && !A_out) return fail(VB_EINVAL, "bias_out needs A_out");
  if (!A_out && !lb && !ub) return fail(VB_EINVAL, "nothing to compute: lb, ub and A_out are NULL");
  if (compact && !alpha) return fail(VB_EINVAL, "a compact layout needs alpha");
  if (alpha) {
    if (!C || ub) return fail(VB_EINVAL, "alpha needs spec rows C and ub == NULL (slopes bound one side)");
    if (compact && (s = check_compact(G, batch, m, compact))) return s;
    for (size_t k = start > stop ? stop + 1 : 0; (int)k < start; ++k)
      if (G.n[k].op == VB_RELU && !alpha[k] && !(compact && compact->width[k] == 0))
        return fail(VB_EINVAL, "alpha of ReLU node %zu is NULL", k);
  }
  {
    // the workspace must hold the weight copies and one batch element's chunk
    // before anything is enqueued (the copies are written first)
    const bool lower_only = C && !ub;
    const long long R = C ? (lower_only ? m : 2LL * m) : 2LL * G.n[start].size;
    const bool plain = !(C || A_out || alpha);
    ChunkPlan plan;
    if ((s = plan_chunks(G, start, stop, R, plain, C != nullptr, 1, ws_bytes, wt_floats(G), plan))) return s;
  }
  return crown_backward_impl(G, batch, start, stop, C, m, node_lo, node_hi, {x_center, x_radius, eps}, lb, ub, ws,
                             ws_bytes, (hipStream_t)stream, A_out, bias_out, alpha, false, compact);
}

extern "C" vb_status vb_concretize(int32_t rows, int32_t n, int32_t rows_per_batch, const float* A, const float* bias,
                                   const float* center, const float* radius, float eps, float* lb, float* ub,
                                   void* stream) {
  if (rows <= 0 || n <= 0 || rows_per_batch <= 0) return fail(VB_EINVAL, "rows, n and rows_per_batch must be > 0");
  if (!A || !center) return fail(VB_EINVAL, "A and center must be non-NULL");
  if (!radius && !(eps >= 0.f)) return fail(VB_EINVAL, "eps must be >= 0");
  HIPCHK(launch_concretize_rows(A, rows, n, rows_per_batch, center, radius, eps, nullptr, nullptr, bias, lb, ub,
                                nullptr, (hipStream_t)stream));
  return VB_OK;
}

extern "C" vb_status vb_crown(const vb_graph* g, int32_t batch, const float* x_center, const float* x_radius,
                              float eps, int32_t method, int32_t region_start, float* const* node_lo,
                              float* const* node_hi, const float* C, int32_t m, float* ibp_lb, float* ibp_ub,
                              float* lb, float* ub, void* ws, size_t ws_bytes, void* stream) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (batch <= 0) return fail(VB_EINVAL, "batch must be positive");
  if ((s = check_domain(x_center))) return s;
  if (!x_radius && !(eps >= 0.f)) return fail(VB_EINVAL, "eps must be >= 0");
  if (!node_lo || !node_hi) return fail(VB_EINVAL, "node_lo/node_hi arrays are NULL");
  const bool intersect = (method & VB_INTERSECT_IBP) != 0;
  const bool unstable_only = (method & VB_UNSTABLE_ONLY) != 0;
  method &= ~(VB_INTERSECT_IBP | VB_UNSTABLE_ONLY);
  if (method < VB_METHOD_IBP || method > VB_METHOD_HYBRID) return fail(VB_EINVAL, "unknown method %d", method);
  if (intersect && method == VB_METHOD_IBP) return fail(VB_EINVAL, "VB_INTERSECT_IBP needs CROWN or HYBRID");
  if (unstable_only && method == VB_METHOD_IBP) return fail(VB_EINVAL, "VB_UNSTABLE_ONLY needs CROWN or HYBRID");
  if (method == VB_METHOD_HYBRID && (region_start <= 0 || region_start >= G.L))
    return fail(VB_EINVAL, "region_start %d out of range", region_start);
  if (C && m <= 0) return fail(VB_EINVAL, "m must be positive with C");
  if (!ws) return fail(VB_EINVAL, "workspace is NULL");
  for (size_t k = 1; k < G.n.size(); ++k)
    if (!node_lo[k] || !node_hi[k]) return fail(VB_EINVAL, "node %zu: bounds storage is NULL", k);
  {
    const size_t need = crown_workspace(G, 1, C ? m : 0, method, region_start, false) +
                        (unstable_only ? 4 * select_floats(G, batch) : 0);
    if (ws_bytes < need)
      return fail(VB_ENOMEM, "workspace of %zu bytes is too small: one batch element needs %zu", ws_bytes, need);
  }
  hipStream_t st = (hipStream_t)stream;
  s = ibp_impl(G, batch, x_center, x_radius, eps, node_lo, node_hi, st, ws, ws_bytes);
  if (s) return s;
  // the weight copies at the head of the workspace serve every backward call below
  if (C || method != VB_METHOD_IBP) {
    std::vector<const float*> wt, beff;
    s = prepare_weights(G, (char*)ws, st, wt, beff);
    if (s) return s;
  }
  if (C && (ibp_lb || ibp_ub)) {
    s = spec_ibp(G, batch, C, m, node_lo, node_hi, ibp_lb, ibp_ub, ws, ws_bytes, st, true);
    if (s) return s;
  }
  const Domain dom{x_center, x_radius, eps};
  int stop = 0;
  if (method != VB_METHOD_IBP) {
    stop = method == VB_METHOD_CROWN ? 0 : region_start;
    for (size_t r = 0; r < G.n.size(); ++r) {
      if (G.n[r].op != VB_RELU) continue;
      const int z = G.n[r].in0;
      if (z <= stop || one_affine_step(G, z, stop)) continue;
      if (unstable_only && G.n[z].op == VB_LINEAR) {
        // rows only for the neurons the bounds so far (IBP) leave unstable, listed on
        // the device (input b's first cnt[b] rows of each sign); the launches cover
        // all n rows per sign and every workgroup whose rows are all past the count
        // returns at once, so nothing is read back
        const long long n = G.n[z].size, nmax = (long long)(select_floats(G, batch) - align_up((size_t)batch * 4) / 4) /
                                                (2 * batch);
        int* idx = (int*)((char*)ws + align_up(wt_floats(G) * 4));
        int* sel = idx + align_up((size_t)batch * nmax * 4) / 4;
        int* cnt = sel + align_up((size_t)batch * nmax * 4) / 4;
        HIPCHK(launch_alpha_layout(node_lo[z], node_hi[z], batch, n, idx, cnt, st));
        HIPCHK(launch_rank_to_list(idx, batch, (int)n, sel, st));
        const int U = (int)n;
        s = crown_backward_impl(G, batch, z, stop, nullptr, 0, node_lo, node_hi, dom, node_lo[z], node_hi[z], ws,
                                ws_bytes, st, nullptr, nullptr, nullptr, intersect, nullptr, true, sel, cnt, U,
                                select_floats(G, batch));
        if (s) return s;
        continue;
      }
      s = crown_backward_impl(G, batch, z, stop, nullptr, 0, node_lo, node_hi, dom, node_lo[z], node_hi[z], ws,
                              ws_bytes, st, nullptr, nullptr, nullptr, intersect, nullptr, true, nullptr, nullptr, 0,
                              unstable_only ? select_floats(G, batch) : 0);
      if (s) return s;
    }
  }
  if (C && (lb || ub)) {
    s = crown_backward_impl(G, batch, G.L, stop, C, m, node_lo, node_hi, dom, lb, ub, ws, ws_bytes, st, nullptr,
                            nullptr, nullptr, false, nullptr, true);
    if (s) return s;
  }
  return VB_OK;
}

extern "C" vb_status vb_verify(int32_t batch, int32_t m, const float* lb, int32_t* verified, int32_t* n_verified,
                               void* stream) {
  if (batch <= 0 || m <= 0) return fail(VB_EINVAL, "batch and m must be positive");
  if (!lb || !verified) return fail(VB_EINVAL, "lb and verified must be non-NULL");
  HIPCHK(launch_verify(lb, batch, m, verified, n_verified, (hipStream_t)stream));
  return VB_OK;
}

extern "C" vb_status vb_crown_noalloc(const vb_graph* g, int32_t batch, const float* x_center,
                                      const float* x_radius, float eps, int32_t method, int32_t region_start,
                                      float* const* node_lo, float* const* node_hi, const float* C, int32_t m,
                                      float* ibp_lb, float* ibp_ub, float* lb, float* ub, void* stream) {
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch((hipStream_t)stream, &ws);
  if (e != hipSuccess) return fail(VB_EDEVICE, "vb_crown_noalloc: scratch address: %s", hipGetErrorString(e));
  const vb_status s = vb_crown(g, batch, x_center, x_radius, eps, method, region_start, node_lo, node_hi, C, m,
                               ibp_lb, ibp_ub, lb, ub, ws, NOALLOC_SCRATCH_BYTES, stream);
  if (s == VB_ENOMEM)
    return fail(VB_ENOMEM, "vb_crown_noalloc: one batch element needs more than the fixed scratch of %zu bytes (%s)",
                NOALLOC_SCRATCH_BYTES, g_err.c_str());
  return s;
}

extern "C" vb_status vb_profile_start(void) {
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  g_prof_on = true;
  return VB_OK;
}

extern "C" vb_status vb_profile_stop(double* ms, double* flops, int64_t* launches) {
  g_prof_on = false;
  double t = 0.0, f = 0.0;
  g_prof_done.clear();
  for (auto& r : g_prof) {
    HIPCHK(hipEventSynchronize(r.b));
    float e = 0.f;
    HIPCHK(hipEventElapsedTime(&e, r.a, r.b));
    t += e;
    f += r.flops;
    ProfDone dn{e, r.flops, {}};
    for (int i = 0; i < 6; ++i) dn.info[i] = r.info[i];
    g_prof_done.push_back(dn);
  }
  if (ms) *ms = t;
  if (flops) *flops = f;
  if (launches) *launches = (int64_t)g_prof.size();
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  return VB_OK;
}

extern "C" vb_status vb_profile_record(int64_t i, double* ms, double* flops, int32_t* info) {
  if (i < 0 || i >= (int64_t)g_prof_done.size()) return fail(VB_EINVAL, "vb_profile_record: no record %lld", (long long)i);
  const ProfDone& r = g_prof_done[(size_t)i];
  if (ms) *ms = r.ms;
  if (flops) *flops = r.flops;
  if (info)
    for (int k = 0; k < 6; ++k) info[k] = r.info[k];
  return VB_OK;
}

// ---------------------------------------------------------------------------
// alpha-CROWN

namespace {

// Affine nodes of a chain network in forward order, each with the ReLU that
// follows it (-1 for the last node).  Returns false if the graph is not a chain.
bool alpha_chain(const Graph& G, std::vector<std::pair<int, int>>& chain) {
  chain.clear();
  for (size_t k = 1; k < G.n.size(); ++k) {
    const NodeInfo& n = G.n[k];
    if (n.op == VB_ADD || n.op == VB_GAP) return false;
    if (n.op != VB_LINEAR && n.op != VB_CONV2D) continue;
    if ((int)k == G.L) {
      chain.push_back({(int)k, -1});
      continue;
    }
    if (n.cons.size() != 1 || G.n[n.cons[0]].op != VB_RELU) return false;
    const int r = n.cons[0];
    // the ReLU feeds exactly one affine node, possibly through flatten
    std::vector<int> c = G.n[r].cons;
    while (c.size() == 1 && G.n[c[0]].op == VB_FLATTEN) c = G.n[c[0]].cons;
    if (c.size() != 1) return false;
    chain.push_back({(int)k, r});
  }
  return !chain.empty() && chain.back().first == G.L && G.n[G.L].op == VB_LINEAR;
}

// kept Psi over the domain and over every ReLU node below `start` (compact:
// width[k] per row)
size_t alpha_psi_floats(const Graph& G, long long rows, const int* width, int start) {
  size_t f = align_up((size_t)rows * G.n[0].size * 4) / 4;
  for (size_t k = 0; k < G.n.size() && (int)k < start; ++k)
    if (G.n[k].op == VB_RELU) f += align_up((size_t)rows * (width ? width[k] : G.n[k].size) * 4) / 4;
  return f;
}

// Workspace of an alpha step on R rows per batch element over node `start`
// (spec rows widen Lambda to the start node).
// The widest ReLU node below `start`.
long long relu_max_size(const Graph& G, int start) {
  long long m = 0;
  for (int k = 0; k < start && k < (int)G.n.size(); ++k)
    if (G.n[k].op == VB_RELU) m = std::max(m, G.n[k].size);
  return m;
}

size_t alpha_workspace_at(const Graph& G, int batch, int start, long long R, bool spec, const int* width,
                          bool with_beta) {
  long long maxw, ppb;
  bwd_requirements(G, start, 0, R, maxw, ppb);
  if (spec) maxw = std::max(maxw, G.n[start].size);
  size_t extra = wt_floats(G) + alpha_psi_floats(G, (long long)batch * R, width, start);
  if (with_beta) extra += align_up((size_t)batch * R * relu_max_size(G, start) * 4) / 4;
  return layout_for(maxw, ppb, R, batch, extra, 0, region_max_size(G, start, 0)).bytes;
}

size_t alpha_workspace(const Graph& G, int batch, int m, const int* width) {
  return alpha_workspace_at(G, batch, G.L, m, true, width, false);
}

}  // namespace

extern "C" vb_status vb_alpha_layout(const vb_graph* g, int32_t batch, const float* const* node_lo,
                                     const float* const* node_hi, int32_t* const* index, int32_t* width, void* ws,
                                     size_t ws_bytes, void* stream) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (batch <= 0) return fail(VB_EINVAL, "batch must be positive");
  if (!node_lo || !node_hi || !index || !width) return fail(VB_EINVAL, "NULL pointer array");
  if (!ws || ws_bytes < (size_t)batch * sizeof(int32_t))
    return fail(VB_ENOMEM, "alpha layout needs %zu bytes of workspace", (size_t)batch * sizeof(int32_t));
  for (size_t k = 0; k < G.n.size(); ++k) {
    if (G.n[k].op != VB_RELU) continue;
    const int z = G.n[k].in0;
    if (!index[k] || !node_lo[z] || !node_hi[z])
      return fail(VB_EINVAL, "ReLU node %zu: index storage / input bounds missing", k);
  }
  hipStream_t st = (hipStream_t)stream;
  int* count = (int*)ws;
  std::vector<int> host(batch);
  for (size_t k = 0; k < G.n.size(); ++k) {
    width[k] = 0;
    if (G.n[k].op != VB_RELU) continue;
    const int z = G.n[k].in0;
    HIPCHK(launch_alpha_layout(node_lo[z], node_hi[z], batch, G.n[z].size, index[k], count, st));
    HIPCHK(hipMemcpyAsync(host.data(), count, (size_t)batch * sizeof(int), hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    width[k] = *std::max_element(host.begin(), host.end());
  }
  return VB_OK;
}

namespace {
// Compact layouts: widths within [0, size], index maps present where a width
// is positive, and every row offset of the state inside 32-bit range.
vb_status check_compact(const Graph& G, int batch, int m, const vb_alpha_compact* c) {
  if (!c->index || !c->width) return fail(VB_EINVAL, "compact layout with NULL index or width array");
  for (size_t k = 0; k < G.n.size(); ++k) {
    if (G.n[k].op != VB_RELU) continue;
    const long long w = c->width[k];
    if (w < 0 || w > G.n[k].size) return fail(VB_EINVAL, "ReLU node %zu: compact width %lld out of range", k, w);
    if (!c->index[k]) return fail(VB_EINVAL, "ReLU node %zu: compact index map is NULL", k);
    if ((long long)batch * m * w >= (1LL << 31))
      return fail(VB_EUNSUPPORTED, "ReLU node %zu: compact state of %lld entries exceeds 2^31", k,
                  (long long)batch * m * w);
  }
  return VB_OK;
}
}  // namespace

extern "C" vb_status vb_alpha_init(const vb_graph* g, int32_t batch, int32_t m, const float* const* node_lo,
                                   const float* const* node_hi, const vb_alpha_compact* compact, float* const* alpha,
                                   float* const* adam_m, float* const* adam_v, void* stream) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (batch <= 0 || m <= 0) return fail(VB_EINVAL, "batch and m must be positive");
  if (!node_lo || !node_hi || !alpha || !adam_m || !adam_v) return fail(VB_EINVAL, "NULL pointer array");
  if (compact && (s = check_compact(G, batch, m, compact))) return s;
  for (size_t k = 0; k < G.n.size(); ++k) {
    if (G.n[k].op != VB_RELU) continue;
    const int z = G.n[k].in0;
    if (!node_lo[z] || !node_hi[z]) return fail(VB_EINVAL, "ReLU node %zu: input bounds missing", k);
    if (compact && compact->width[k] == 0) continue;  // no unstable neuron: no state
    if (!alpha[k]) continue;                          // a node this state does not cover
    if (!adam_m[k] || !adam_v[k]) return fail(VB_EINVAL, "ReLU node %zu: adam state missing", k);
  }
  for (size_t k = 0; k < G.n.size(); ++k) {
    if (G.n[k].op != VB_RELU || !alpha[k]) continue;
    const int z = G.n[k].in0;
    const int* aidx = compact ? compact->index[k] : nullptr;
    const int acols = compact ? compact->width[k] : 0;
    HIPCHK(launch_alpha_init(node_lo[z], node_hi[z], batch, m, G.n[z].size, aidx, acols, alpha[k], adam_m[k],
                             adam_v[k], (hipStream_t)stream));
  }
  return VB_OK;
}

extern "C" vb_status vb_alpha_step_rows(const vb_graph* g, int32_t batch, int32_t start, const float* C, int32_t m,
                                        const float* const* node_lo, const float* const* node_hi,
                                        const float* x_center, const float* x_radius, float eps,
                                        const vb_alpha_compact* compact, const vb_beta* beta, float* const* alpha,
                                        float* const* adam_m, float* const* adam_v, int32_t step, float lr,
                                        float beta1, float beta2,
                                        float adam_eps, float* lb_out, float* best_lb, float* ub_out, float* best_ub,
                                        void* ws, size_t ws_bytes, void* stream) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (batch <= 0) return fail(VB_EINVAL, "batch must be positive");
  if (start <= 0 || start >= (int)G.n.size() || (G.n[start].op != VB_LINEAR && G.n[start].op != VB_CONV2D))
    return fail(VB_EINVAL, "start %d must be a Linear or Conv node", start);
  if (C && m <= 0) return fail(VB_EINVAL, "m must be positive with C");
  if (C && (ub_out || best_ub)) return fail(VB_EINVAL, "spec rows bound one side: ub_out / best_ub must be NULL");
  const bool ident = C == nullptr;
  const long long R = ident ? 2LL * G.n[start].size : m;
  if ((s = check_domain(x_center))) return s;
  if (!x_radius && !(eps >= 0.f)) return fail(VB_EINVAL, "eps must be >= 0");
  if (!node_lo || !node_hi || !alpha) return fail(VB_EINVAL, "NULL pointer array");
  if (step < 0) return fail(VB_EINVAL, "step must be >= 0");
  if (step > 0 && (!adam_m || !adam_v)) return fail(VB_EINVAL, "Adam state arrays are NULL");
  if (!(lr >= 0.f) || !(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(adam_eps > 0.f))
    return fail(VB_EINVAL, "bad Adam hyper-parameters");
  if (!lb_out && !best_lb && !ub_out && !best_ub) return fail(VB_EINVAL, "no output: lb_out, best_lb (ub_out, best_ub) NULL");
  if ((long long)batch * R >= (1LL << 31)) return fail(VB_EUNSUPPORTED, "batch x rows beyond 2^31");
  std::vector<std::pair<int, int>> chain;
  if (!alpha_chain(G, chain)) return fail(VB_EUNSUPPORTED, "alpha-CROWN needs a chain of Linear/Conv + ReLU nodes");
  if (compact && (s = check_compact(G, batch, (int)R, compact))) return s;
  if (beta) {
    if (compact) return fail(VB_EUNSUPPORTED, "split constraints need the dense alpha layout");
    if (!beta->split || !beta->beta) return fail(VB_EINVAL, "beta state with NULL split or beta arrays");
    if (step > 0 && (!beta->beta_m || !beta->beta_v)) return fail(VB_EINVAL, "beta Adam state arrays are NULL");
    for (size_t k = 0; k < G.n.size() && (int)k < start; ++k)
      if (G.n[k].op == VB_RELU && beta->split[k] &&
          (!beta->beta[k] || (step > 0 && (!beta->beta_m[k] || !beta->beta_v[k]))))
        return fail(VB_EINVAL, "ReLU node %zu: split without beta / beta Adam state", k);
  }
  for (size_t k = 0; k < G.n.size() && (int)k < start; ++k) {
    if (G.n[k].op != VB_RELU) continue;
    const int z = G.n[k].in0;
    if (!node_lo[z] || !node_hi[z]) return fail(VB_EINVAL, "ReLU node %zu: input bounds missing", k);
    if (compact && compact->width[k] == 0) continue;  // no unstable neuron: no state
    if (!alpha[k] || (step > 0 && (!adam_m[k] || !adam_v[k])))
      return fail(VB_EINVAL, "ReLU node %zu: alpha / adam state missing", k);
  }
  if (!ws) return fail(VB_EINVAL, "workspace is NULL");
  const size_t need = alpha_workspace_at(G, batch, start, R, !ident, compact ? compact->width : nullptr, beta != nullptr);
  if (ws_bytes < need)
    return fail(VB_ENOMEM, "alpha step needs %zu bytes of workspace for the whole batch (got %zu)", need, ws_bytes);
  hipStream_t st = (hipStream_t)stream;
  const long long rows = (long long)batch * R;

  // workspace: [transposed weights][kept psi per ReLU + domain][backward pool ...]
  char* base = (char*)ws;
  Backward B{G, st, node_lo, node_hi, {x_center, x_radius, eps}};
  s = prepare_weights(G, base, st, B.wt, B.beff);
  if (s) return s;
  size_t off = align_up(wt_floats(G) * 4);
  std::vector<float*> psi(G.n.size(), nullptr);
  psi[0] = (float*)(base + off);
  off += align_up((size_t)rows * G.n[0].size * 4);
  for (size_t k = 0; k < G.n.size() && (int)k < start; ++k)
    if (G.n[k].op == VB_RELU) {
      const long long w = compact ? compact->width[k] : G.n[k].size;
      psi[k] = w > 0 ? (float*)(base + off) : nullptr;
      off += align_up((size_t)rows * w * 4);
    }
  // (a compact node without unstable neurons has no state: its slopes are never read)
  std::vector<const float*> al(G.n.size(), nullptr);
  for (size_t k = 0; k < G.n.size() && (int)k < start; ++k)
    al[k] = (compact && G.n[k].op == VB_RELU && compact->width[k] == 0) ? nullptr : alpha[k];
  B.alpha = al.data();
  B.psi_keep = psi.data();
  B.beta = beta;
  // adjoint over a split ReLU input (beta's gradient), [rows][widest ReLU node]
  float* gzbuf = nullptr;
  if (beta) {
    gzbuf = (float*)(base + off);
    off += align_up((size_t)rows * relu_max_size(G, start) * 4);
  }
  if (compact) {
    B.aidx = compact->index;
    B.awidth = compact->width;
  }
  // evaluation: lower bounds of the rows with the current slopes (identity rows:
  // +e_j gives l_j, -e_j gives -u_j)
  const int n = (int)G.n[start].size;
  s = backward_all(B, start, 0, C, m, ident ? 1 : 0, batch, R, base, ws_bytes, off / 4,
                   [&](float* acc, int b0, int cb) -> vb_status {
                     if (b0 != 0 || cb != batch) return fail(VB_ENOMEM, "internal: alpha step was chunked");
                     if (!ident) {
                       HIPCHK(launch_finish_lower(acc, rows, lb_out, best_lb, step == 1, st));
                     } else {
                       if (lb_out || ub_out) HIPCHK(launch_finish(acc, batch, n, lb_out, ub_out, nullptr, st, 0));
                       if (best_lb || best_ub)
                         HIPCHK(launch_finish(acc, batch, n, best_lb, best_ub, nullptr, st, step == 1 ? 0 : 1));
                     }
                     return VB_OK;
                   });
  if (s) return s;
  if (step == 0) return VB_OK;

  // adjoint, forward through the chain; the evaluation's pool buffers are free now
  float* gbuf[2] = {B.pool[0], B.pool[1]};
  HIPCHK(launch_adj_domain(psi[0], (int)rows, (int)G.n[0].size, (int)R, x_center, x_radius, eps, gbuf[0], st));
  const double bc1 = 1.0 / (1.0 - std::pow((double)beta1, step));
  const double bc2 = 1.0 / (1.0 - std::pow((double)beta2, step));
  int cur = 0;
  for (const auto& kr : chain) {
    const int k = kr.first, r = kr.second;
    if (r < 0 || k >= start) break;  // the start node: its adjoint is not needed
    const NodeInfo& nd = G.n[k];
    const NodeInfo& in = G.n[src_of(G, nd.in0)];
    GemmDesc d = affine_forward(nd, in, (int)rows);
    d.A = gbuf[cur];
    ConvAdj ca{};
    if (nd.op == VB_CONV2D) {
      ca.g0 = gbuf[cur];
      ca.W = nd.W;
      ca.Ci = in.c;
      ca.Hi = in.h;
      ca.Wi = in.w;
      ca.Co = nd.c;
      ca.Ho = nd.h;
      ca.Wo = nd.w;
      ca.kh = nd.kh;
      ca.kw = nd.kw;
      ca.stride = nd.stride;
      ca.pad = nd.pad;
    }
    // few input channels: a direct kernel when it takes the shape, else an
    // im2col image and a GEMM over it
    const bool direct = nd.op == VB_CONV2D && conv_adjoint_fits(ca);
    const int Kp = (nd.kh * nd.kw * in.c + 31) / 32 * 32;
    if (!direct && nd.op == VB_CONV2D && in.c % 32 != 0 && (size_t)rows * nd.h * nd.w * Kp <= B.pool_floats &&
        (size_t)nd.c * Kp <= B.pool_floats) {
      // few input channels: im2col of the adjoint, then a 1x1 conv over that image
      // with K padded to whole 32-deep stages (the GEMM's fast path)
      HIPCHK(launch_im2col(gbuf[cur], (int)rows, in.h, in.w, in.c, nd.kh, nd.kw, nd.stride, nd.pad, nd.h, nd.w, Kp,
                           B.pool[2], st));
      HIPCHK(launch_pad_weights(nd.W, nd.kh * nd.kw, nd.c, in.c, Kp, B.pool[3], st));
      NodeInfo n1 = nd, i1 = in;
      n1.kh = n1.kw = n1.stride = 1;
      n1.pad = 0;
      i1.c = Kp;
      i1.h = nd.h;
      i1.w = nd.w;
      i1.size = (long long)nd.h * nd.w * Kp;
      d = affine_forward(n1, i1, (int)rows);
      d.A = B.pool[2];
      d.B = B.pool[3];
    }
    d.epi = E_ADJOINT;
    d.amode = A_PLAIN;
    d.out = gbuf[cur ^ 1];
    d.bias = nd.b;
    d.bias_c = 0;
    // coefficient buffer of the evaluation's layout: 4 * batch * (widest node) floats
    HIPCHK(launch_relax_coef(node_lo[k], node_hi[k], (long long)batch * nd.size,
                             compact ? compact->index[r] : nullptr, B.coef, st));
    d.coef = B.coef;
    d.rows_per_b = (int)R;
    const bool none = compact && compact->width[r] == 0;
    d.psi_in = psi[r];
    d.alpha_rw = none ? nullptr : alpha[r];
    d.adam_m = none ? nullptr : adam_m[r];
    d.adam_v = none ? nullptr : adam_v[r];
    d.aidx = compact ? compact->index[r] : nullptr;
    d.acols = compact ? compact->width[r] : 0;
    d.do_update = 1;
    d.lr = lr;
    d.beta1 = beta1;
    d.beta2 = beta2;
    d.bc1 = (float)bc1;
    d.bc2 = (float)bc2;
    d.adam_eps = adam_eps;
    AdjFinish a{};
    a.rows_per_b = d.rows_per_b;
    a.bias = d.bias;
    a.coef = d.coef;
    a.psi_in = d.psi_in;
    a.alpha_rw = d.alpha_rw;
    a.adam_m = d.adam_m;
    a.adam_v = d.adam_v;
    a.aidx = d.aidx;
    a.acols = d.acols;
    a.do_update = d.do_update;
    a.lr = d.lr;
    a.beta1 = d.beta1;
    a.beta2 = d.beta2;
    a.bc1 = d.bc1;
    a.bc2 = d.bc2;
    a.adam_eps = d.adam_eps;
    a.out = d.out;
    const bool split_here = beta && beta->split[r] && gzbuf;
    if (split_here) {
      d.gz_out = gzbuf;
      a.gz_out = gzbuf;
    }
    auto beta_update = [&]() -> vb_status {
      if (!split_here) return VB_OK;
      HIPCHK(launch_beta_adam((int)rows, (int)R, (int)nd.size, gzbuf, beta->split[r], beta->beta[r], beta->beta_m[r],
                              beta->beta_v[r], lr, beta1, beta2, (float)bc1, (float)bc2, adam_eps, st));
      return VB_OK;
    };
    if (direct) {
      ca.a = a;
      ca.a.M = (int)rows;
      ca.a.N = (int)nd.size;
      HIPCHK(launch_conv_adjoint_first(ca, (int)rows, st));
      if ((s = beta_update())) return s;
      cur ^= 1;
      continue;
    }
    const int S = gemm_is_dense(d) ? ibp_gemm_split(d) : 1;
    if (S > 1 && (size_t)S * d.M * d.N <= B.pool_floats) {
      // few output tiles (a Linear over batch x specs rows): split K, then
      // apply the adjoint epilogue to the summed slices
      GemmDesc e = d;
      e.ksplit = S;
      e.out = B.pool[2];
      HIPCHK(launch_gemm(e, st));
      a.part = B.pool[2];
      a.S = S;
      a.M = d.M;
      a.N = d.N;
      HIPCHK(launch_adjoint_finish(a, st));
    } else {
      HIPCHK(launch_gemm(d, st));
    }
    if ((s = beta_update())) return s;
    cur ^= 1;
  }
  return VB_OK;
}

extern "C" vb_status vb_alpha_step(const vb_graph* g, int32_t batch, const float* C, int32_t m,
                                   const float* const* node_lo, const float* const* node_hi, const float* x_center,
                                   const float* x_radius, float eps, const vb_alpha_compact* compact,
                                   float* const* alpha, float* const* adam_m, float* const* adam_v, int32_t step,
                                   float lr, float beta1, float beta2, float adam_eps, float* lb_out, float* best_lb,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!C) return fail(VB_EINVAL, "C is NULL");
  if (!g || !g->nodes || g->n_nodes < 2) return fail(VB_EINVAL, "graph is NULL or has fewer than 2 nodes");
  return vb_alpha_step_rows(g, batch, g->n_nodes - 1, C, m, node_lo, node_hi, x_center, x_radius, eps, compact,
                            nullptr, alpha, adam_m, adam_v, step, lr, beta1, beta2, adam_eps, lb_out, best_lb, nullptr,
                            nullptr, ws, ws_bytes, stream);
}

extern "C" vb_status vb_apply_splits(const vb_graph* g, int32_t batch, const float* const* split,
                                     float* const* node_lo, float* const* node_hi, void* stream) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (batch <= 0) return fail(VB_EINVAL, "batch must be positive");
  if (!split || !node_lo || !node_hi) return fail(VB_EINVAL, "NULL pointer array");
  for (size_t k = 0; k < G.n.size(); ++k)
    if (G.n[k].op == VB_RELU && split[k] && (!node_lo[G.n[k].in0] || !node_hi[G.n[k].in0]))
      return fail(VB_EINVAL, "ReLU node %zu: bounds of its input missing", k);
  for (size_t k = 0; k < G.n.size(); ++k) {
    if (G.n[k].op != VB_RELU || !split[k]) continue;
    const int z = G.n[k].in0;
    HIPCHK(launch_apply_splits(split[k], (long long)batch * G.n[z].size, node_lo[z], node_hi[z], (hipStream_t)stream));
  }
  return VB_OK;
}

namespace {
// Workspace carve-up of the branch-and-bound driver for `D` sub-domains at a time.
struct BabLayout {
  std::vector<size_t> lo, hi;        // per node: domain bounds [D][size]
  size_t x, rad, C;                  // replicated input box and spec rows
  std::vector<size_t> split, score;  // per ReLU node: [D][size]
  std::vector<size_t> al, am, av, be, bm, bv;  // per ReLU node: [D][m][size]
  size_t lb, best;                   // [D][m]
  size_t step_ws, step_bytes;        // the alpha-beta step's own workspace
  size_t bytes;
};

BabLayout bab_layout(const Graph& G, int m, int D) {
  BabLayout L;
  const size_t N = G.n.size();
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t o = off;
    off += align_up(floats * 4);
    return o;
  };
  L.lo.assign(N, 0);
  L.hi.assign(N, 0);
  L.split.assign(N, 0);
  L.score.assign(N, 0);
  L.al.assign(N, 0);
  L.am.assign(N, 0);
  L.av.assign(N, 0);
  L.be.assign(N, 0);
  L.bm.assign(N, 0);
  L.bv.assign(N, 0);
  for (size_t k = 1; k < N; ++k) {
    L.lo[k] = take((size_t)D * G.n[k].size);
    L.hi[k] = take((size_t)D * G.n[k].size);
  }
  L.x = take((size_t)D * G.n[0].size);
  L.rad = take((size_t)D * G.n[0].size);
  L.C = take((size_t)D * m * G.n[G.L].size);
  for (size_t k = 0; k < N; ++k) {
    if (G.n[k].op != VB_RELU) continue;
    const size_t n = (size_t)G.n[k].size;
    L.split[k] = take((size_t)D * n);
    L.score[k] = take((size_t)D * n);
    for (auto* v : {&L.al, &L.am, &L.av, &L.be, &L.bm, &L.bv}) (*v)[k] = take((size_t)D * m * n);
  }
  L.lb = take((size_t)D * m);
  L.best = take((size_t)D * m);
  L.step_ws = off;
  L.step_bytes = alpha_workspace_at(G, D, G.L, m, true, nullptr, true);
  L.bytes = off + L.step_bytes;
  return L;
}

struct SplitRec {
  int node, idx;
  float sign;
};
}  // namespace

extern "C" vb_status vb_bab_workspace_size(const vb_graph* g, int32_t m, int32_t batch, size_t* bytes) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (!bytes || m <= 0 || batch <= 0) return fail(VB_EINVAL, "m and batch must be positive, bytes non-NULL");
  std::vector<std::pair<int, int>> chain;
  if (!alpha_chain(G, chain)) return fail(VB_EUNSUPPORTED, "branch and bound needs a chain of Linear/Conv + ReLU nodes");
  *bytes = bab_layout(G, m, batch).bytes;
  return VB_OK;
}

extern "C" vb_status vb_bab(const vb_graph* g, const float* x_center, const float* x_radius, float eps,
                            const float* C, int32_t m, const float* const* node_lo, const float* const* node_hi,
                            const vb_bab_params* p, int32_t* verdict, int32_t* domains, float* root_lb, void* ws,
                            size_t ws_bytes, void* stream) {
  Graph G;
  vb_status s = parse_graph(g, G);
  if (s) return s;
  if (!p || !verdict || !domains) return fail(VB_EINVAL, "params, verdict and domains must be non-NULL");
  if (!C || m <= 0) return fail(VB_EINVAL, "C must be non-NULL and m positive");
  if ((s = check_domain(x_center))) return s;
  if (!x_radius && !(eps >= 0.f)) return fail(VB_EINVAL, "eps must be >= 0");
  if (!node_lo || !node_hi) return fail(VB_EINVAL, "NULL pointer array");
  if (p->steps < 1 || p->batch < 1 || p->max_domains < 1) return fail(VB_EINVAL, "steps, batch and max_domains must be >= 1");
  if (!(p->lr >= 0.f) || !(p->beta1 >= 0.f && p->beta1 < 1.f) || !(p->beta2 >= 0.f && p->beta2 < 1.f) ||
      !(p->adam_eps > 0.f))
    return fail(VB_EINVAL, "bad Adam hyper-parameters");
  std::vector<std::pair<int, int>> chain;
  if (!alpha_chain(G, chain)) return fail(VB_EUNSUPPORTED, "branch and bound needs a chain of Linear/Conv + ReLU nodes");
  for (size_t k = 1; k < G.n.size(); ++k)
    if (!node_lo[k] || !node_hi[k]) return fail(VB_EINVAL, "node %zu: root bounds missing", k);
  if (!ws) return fail(VB_EINVAL, "workspace is NULL");
  const int D = p->batch;
  const BabLayout L = bab_layout(G, m, D);
  if (ws_bytes < L.bytes)
    return fail(VB_ENOMEM, "branch and bound needs %zu bytes of workspace (got %zu)", L.bytes, ws_bytes);
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  const size_t N = G.n.size();
  auto F = [&](size_t off) { return (float*)(base + off); };
  std::vector<float*> lo(N, nullptr), hi(N, nullptr), split(N, nullptr), al(N, nullptr), am(N, nullptr),
      av(N, nullptr), be(N, nullptr), bm(N, nullptr), bv(N, nullptr), score(N, nullptr);
  std::vector<int> relus;
  for (size_t k = 1; k < N; ++k) {
    lo[k] = F(L.lo[k]);
    hi[k] = F(L.hi[k]);
  }
  for (size_t k = 0; k < N; ++k)
    if (G.n[k].op == VB_RELU) {
      relus.push_back((int)k);
      split[k] = F(L.split[k]);
      score[k] = F(L.score[k]);
      al[k] = F(L.al[k]);
      am[k] = F(L.am[k]);
      av[k] = F(L.av[k]);
      be[k] = F(L.be[k]);
      bm[k] = F(L.bm[k]);
      bv[k] = F(L.bv[k]);
    }
  const long long n0 = G.n[0].size, nL = G.n[G.L].size;
  HIPCHK(launch_broadcast(x_center, n0, D, F(L.x), st));
  if (x_radius) HIPCHK(launch_broadcast(x_radius, n0, D, F(L.rad), st));
  HIPCHK(launch_broadcast(C, (long long)m * nL, D, F(L.C), st));
  const vb_beta bst{split.data(), be.data(), bm.data(), bv.data()};

  std::vector<std::vector<SplitRec>> queue(1);
  size_t head = 0;
  int processed = 0;
  bool stopped = false;
  std::vector<float> hsplit, hbest((size_t)D * m), hscore;
  while (head < queue.size()) {
    if (processed >= p->max_domains) {
      stopped = true;
      break;
    }
    const int nd = (int)std::min<size_t>((size_t)D, queue.size() - head);
    // this round's split arrays (host, every ReLU node's in one buffer, copied
    // with one wait for all of them), then the clamped bounds of every sub-domain
    {
      size_t total = 0;
      for (int r : relus) total += (size_t)nd * G.n[r].size;
      hsplit.assign(total, 0.f);
      size_t at = 0;
      for (int r : relus) {
        const long long n = G.n[r].size;
        float* h = hsplit.data() + at;
        for (int i = 0; i < nd; ++i)
          for (const SplitRec& q : queue[head + i])
            if (q.node == r) h[(size_t)i * n + q.idx] = q.sign;
        HIPCHK(hipMemcpyAsync(split[r], h, (size_t)nd * n * 4, hipMemcpyHostToDevice, st));
        at += (size_t)nd * n;
      }
      HIPCHK(hipStreamSynchronize(st));  // (the host buffer is reused next round)
    }
    for (size_t k = 1; k < N; ++k) {
      HIPCHK(launch_broadcast(node_lo[k], G.n[k].size, nd, lo[k], st));
      HIPCHK(launch_broadcast(node_hi[k], G.n[k].size, nd, hi[k], st));
    }
    for (int r : relus) {
      const int z = G.n[r].in0;
      HIPCHK(launch_apply_splits(split[r], (long long)nd * G.n[z].size, lo[z], hi[z], st));
      HIPCHK(launch_alpha_init(lo[z], hi[z], nd, m, G.n[z].size, nullptr, 0, al[r], am[r], av[r], st));
      HIPCHK(launch_fill(be[r], 0.f, (long long)nd * m * G.n[r].size, st));
      HIPCHK(launch_fill(bm[r], 0.f, (long long)nd * m * G.n[r].size, st));
      HIPCHK(launch_fill(bv[r], 0.f, (long long)nd * m * G.n[r].size, st));
    }
    // alpha-beta-CROWN on the spec rows of every sub-domain, then one evaluation
    for (int t = 1; t <= p->steps + 1; ++t) {
      const int step = t <= p->steps ? t : 0;
      s = vb_alpha_step_rows(g, nd, G.L, F(L.C), m, lo.data(), hi.data(), F(L.x), x_radius ? F(L.rad) : nullptr,
                             eps, nullptr, &bst, al.data(), am.data(), av.data(), step, p->lr, p->beta1, p->beta2,
                             p->adam_eps, F(L.lb), F(L.best), nullptr, nullptr, base + L.step_ws, L.step_bytes,
                             stream);
      if (s) return s;
    }
    if (head == 0 && root_lb) HIPCHK(hipMemcpyAsync(root_lb, F(L.best), (size_t)m * 4, hipMemcpyDeviceToDevice, st));
    // branching scores from the last evaluation's Psi over each ReLU (kept in the
    // step's workspace: after the weight copies and the domain's Psi)
    {
      const long long rows = (long long)nd * m;
      size_t off = align_up(wt_floats(G) * 4) + align_up((size_t)rows * n0 * 4);
      for (size_t k = 0; k < N && (int)k < G.L; ++k) {
        if (G.n[k].op != VB_RELU) continue;
        const float* psi = (const float*)(base + L.step_ws + off);
        off += align_up((size_t)rows * G.n[k].size * 4);
        const int z = G.n[k].in0;
        HIPCHK(launch_branch_score(psi, F(L.best), nd, m, (int)G.n[k].size, lo[z], hi[z], score[k], st));
      }
    }
    HIPCHK(hipMemcpyAsync(hbest.data(), F(L.best), (size_t)nd * m * 4, hipMemcpyDeviceToHost, st));
    hscore.clear();
    std::vector<size_t> soff(N, 0);
    for (int r : relus) {
      soff[r] = hscore.size();
      hscore.resize(hscore.size() + (size_t)nd * G.n[r].size);
    }
    for (int r : relus)
      HIPCHK(hipMemcpyAsync(hscore.data() + soff[r], score[r], (size_t)nd * G.n[r].size * 4, hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    std::vector<std::vector<SplitRec>> children;
    for (int i = 0; i < nd && !stopped; ++i) {
      ++processed;
      bool proved = true;
      for (int r = 0; r < m; ++r) proved = proved && hbest[(size_t)i * m + r] > 0.f;
      if (proved) continue;
      // the neuron with the largest score (ties: lowest node, then lowest index)
      int bn = -1, bi = -1;
      float bs = -INFINITY;
      for (int r : relus) {
        const long long n = G.n[r].size;
        for (long long j = 0; j < n; ++j) {
          const float v = hscore[soff[r] + (size_t)i * n + j];
          if (v == -INFINITY) continue;
          if (bn < 0 || v > bs) {
            bn = r;
            bi = (int)j;
            bs = v;
          }
        }
      }
      if (bn < 0) {
        stopped = true;  // no unstable neuron left: the search cannot refine this sub-domain
        break;
      }
      for (float sign : {1.f, -1.f}) {
        std::vector<SplitRec> child = queue[head + i];
        child.push_back({bn, bi, sign});
        children.push_back(std::move(child));
      }
    }
    if (stopped) break;
    head += nd;
    for (auto& c : children) queue.push_back(std::move(c));
  }
  *verdict = stopped ? 0 : 1;
  *domains = processed;
  return VB_OK;
}

// ---------------------------------------------------------------------------
// host-only helpers for the tests (vb_testing.h)

#include "vb_testing.h"

extern "C" int32_t vb_testing_fastdiv(int32_t d, const int32_t* x, int64_t n, int32_t* q, uint32_t* mul,
                                      uint32_t* shr) {
  if (d < 1 || n < 0 || (n > 0 && (!x || !q))) return -1;
  const FastDiv f = make_fastdiv(d);
  if (mul) *mul = f.mul;
  if (shr) *shr = f.shr;
  for (int64_t i = 0; i < n; ++i) {
    if (x[i] < 0) return -1;
    // the kernels' division: high 32 bits of x * mul, shifted right by shr
    q[i] = f.d == 1 ? x[i] : (int32_t)((uint32_t)(((uint64_t)(uint32_t)x[i] * f.mul) >> 32) >> f.shr);
  }
  return 0;
}

extern "C" int32_t vb_testing_conv_tile_n(int32_t mode, int32_t rows, int32_t h, int32_t w, int32_t c_in,
                                          int32_t c_out) {
  if (rows <= 0 || h <= 0 || w <= 0 || c_in <= 0 || c_out <= 0) return -1;
  NodeInfo in{}, nd{};
  in.op = VB_RELU;
  in.c = c_in;
  in.h = h;
  in.w = w;
  in.size = (long long)c_in * h * w;
  nd.op = VB_CONV2D;
  nd.c = c_out;
  nd.h = h;
  nd.w = w;
  nd.size = (long long)c_out * h * w;
  nd.kh = nd.kw = 3;
  nd.stride = 1;
  nd.pad = 1;
  // stand-in operand addresses: only their alignment is looked at, nothing is read
  const float* fake = reinterpret_cast<const float*>((uintptr_t)4096);
  nd.W = fake;
  GemmDesc d;
  if (mode == E_STORE || mode == E_RELAX || mode == E_CONCRETIZE) {
    if (!conv_backward(nd, in, fake, rows, 0, 0, d)) return -1;
  } else if (mode == E_ADJOINT) {
    d = affine_forward(nd, in, rows);
    d.A = fake;
  } else {
    return -1;
  }
  d.epi = mode;
  d.B = fake;
  const int nt = gemm_ntiles(d);
  if (nt <= 0) return -1;
  // the narrowest of the launcher's widths that covers N with nt tiles
  for (int bn : {32, 64, 128, 256})
    if ((d.N + bn - 1) / bn == nt) return bn;
  return -1;
}

extern "C" int32_t vb_testing_identity_path(const vb_graph* g, int32_t start, int32_t stop) {
  Graph G;
  if (parse_graph(g, G) != VB_OK) return -1;
  if (start <= 0 || start >= (int)G.n.size() || stop < 0 || stop >= start) return -1;
  std::vector<PatchStep> steps;
  if (patch_chain_graph(G, start, stop, steps)) return 1;
  std::vector<Win> W;
  std::vector<char> active;
  if (window_plan(G, start, stop, W, active)) return 2;
  return 0;
}

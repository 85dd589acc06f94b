// Internal interface between the host planner (vb_api.cpp) and the HIP kernels
// (vb_gemm.hip, vb_kernels.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <cstdint>

namespace vb {

// How the A operand of the implicit GEMM is read.
enum AMode : int {
  A_PLAIN = 0,     // A values as stored
  A_IBP_BOX = 1,   // A = lo, A2 = hi: operands c = (lo+hi)/2 and r = (hi-lo)/2
  A_IBP_BALL = 2,  // A = centre, A2 = radius array or NULL (scalar eps): c and r
};

// What the GEMM epilogue does with each output element v = acc (+ addend).
enum EpiMode : int {
  E_STORE = 0,       // out = v; row partial += v . bias (if bias)
  E_RELAX = 1,       // out = v>=0 ? a v : s v with (a,s,t) from target bounds;
                     // row partial += out . bias + min(v,0) t
  E_CONCRETIZE = 2,  // row partial += v c - |v| r over the domain box
  E_IBP = 3,         // lo = acc_c + bias - acc_r, hi = acc_c + bias + acc_r
  E_ADJOINT = 4,     // alpha-CROWN adjoint through a ReLU: g = acc + bias over z;
                     // d(sum lb)/d alpha = g * max(psi, 0) on unstable neurons ->
                     // Adam ascent on alpha (in place); out = g * (psi>=0 ? alpha_old : s)
                     // + (psi<0 ? t : 0)
};

constexpr int MAX_TAPS = 9;

// Division by a runtime constant d >= 1 for 0 <= x < 2^31 by multiply-high:
// with l = ceil(log2 d), mul = ceil(2^(31+l) / d) (< 2^32), x / d =
// umulhi(x, mul) >> (l - 1); exact because x * (mul - 2^(31+l)/d) / 2^(31+l)
// < 2^-l <= 1/d.  d = 1 is passed through (mul = 0).
struct FastDiv {
  uint32_t mul;
  uint32_t shr;
  int32_t d;
};
inline FastDiv make_fastdiv(int d) {
  FastDiv f{0u, 0u, d};
  if (d > 1) {
    uint32_t l = 0;
    while ((1ull << l) < (unsigned long long)d) ++l;
    f.mul = (uint32_t)(((1ull << (31 + l)) + (unsigned long long)d - 1) / (unsigned long long)d);
    f.shr = l - 1;
  }
  return f;
}

struct GemmDesc {
  int M, N, K;                 // output positions x output channels x reduction length
  int amode;                   // AMode of the A operand (E_IBP: A_IBP_BOX or A_IBP_BALL)
  // ---- A operand: position m -> (row, Y, X) on a gh x gw grid per row; for a
  //      gather (conv) GEMM, M = rows * gh * gw and the tiles walk a padded
  //      index space of blocks of 2^rb_shift rows: m = (rb*gh*gw + Y*gw + X) *
  //      2^rb_shift + (row mod 2^rb_shift), rb = row >> rb_shift.  A tile thus
  //      holds a few rows at a few neighbouring pixels (their relaxation data is
  //      shared), and consecutive tiles sweep one block of rows over all pixels,
  //      so the neighbouring pixels that the taps read are still in L2;
  //      reduction index k -> (tap j, channel c) with k = j*cs + c;
  //      element = A[row*a_row_stride + ((Y*sy + dy_j)*ws + (X*sx + dx_j))*cs + c],
  //      zero outside [0,hs) x [0,ws).  Dense GEMM: gh=gw=hs=ws=1, cs=K, 1 tap.
  const float* A;              // A_IBP_BOX: lo;  A_IBP_BALL: centre
  const float* A2;             // A_IBP_BOX: hi;  A_IBP_BALL: radius array or NULL (eps)
  float eps;
  int gh, gw, hs, ws, cs, sy, sx;
  long long a_row_stride;
  int ntaps;
  int tap_dy[MAX_TAPS], tap_dx[MAX_TAPS], tap_w[MAX_TAPS];
  // ---- B operand (weights), tap-major and K-contiguous: k = j*cs + c,
  //      element (k, n) = B[(tap_w[j]*N + n)*cs + c]
  const float* B;
  // ---- output mapping: (row, Y, X) -> row*ho*wo + (Y*oym+oy0)*wo + (X*oxm+ox0)
  int ho, wo, oym, oy0, oxm, ox0;
  int rows_per_b;              // batch element of a row = row / rows_per_b
  FastDiv div_p, div_gw, div_rows, div_nrows;  // filled by launch_gemm: gh*gw, gw, rows_per_b, M/(gh*gw)
  // ---- footprint (patch) mode of a gather GEMM: the rows are identity rows
  //      (b, sign, p, c) over a node of pgh x pgw pixels and pc channels, and
  //      Lambda lives on a window of the target node: output cell (Y, X) of
  //      row p = (py, px) is the target's pixel (py*psy + poy + Y, px*psx +
  //      pox + X) of an img_h x img_w grid.  Cells outside that grid take no
  //      relaxation (zero) and no domain.
  int patch;
  FastDiv div_pc, div_pz, div_pw;  // filled by launch_gemm: pc, pgh*pgw, pgw
  int pc, pgh, pgw, psy, poy, psx, pox, img_h, img_w;
  //      and of the A operand's window: source cell (Ys, Xs) of row p is pixel
  //      (py*ssy + soy + Ys, px*ssx + sox + Xs) of a src_h x src_w node
  //      (src_h = 0: not given; then only the window's own bounds are known)
  int ssy, soy, ssx, sox, src_h, src_w;
  //      a second A source (footprint windows, concretisation): taps j >=
  //      tap_src1 read Lambda A1 (row stride a1_row_stride) on its own
  //      hs1 x ws1 window grid, whose cell (Ys, Xs) for row p is pixel
  //      (py*ssy1 + soy1 + Ys, px*ssx1 + sox1 + Xs) of a src_h1 x src_w1 node,
  //      with weights B1 (same [tap][N][cs] layout, tap_w indexing B1).  The
  //      two sources' products land on the same output window and are summed
  //      by the reduction itself.  A1 == NULL: every tap reads A.
  const float* A1;
  const float* B1;
  long long a1_row_stride;
  int tap_src1, hs1, ws1, ssy1, soy1, ssx1, sox1, src_h1, src_w1;
  // rows of selected neurons (unstable-only identity rows): row r of batch element
  // b = r / (2 live_u) is live iff (r mod live_u) < live_cnt[b]; a workgroup whose
  // rows are all dead returns at once (their outputs and partials are never read)
  const int* live_cnt;
  int live_u;
  int Mt;                      // filled by launch_gemm: size of the tile index space (gather: padded)
  int rb_shift;                // filled by launch_gemm: log2 of the rows per block (gather)
  // ---- epilogue
  int epi;
  float* out;                  // [opos][N]   (E_IBP: lo)
  float* out2;                 // E_IBP: hi
  float* relu_lo;              // E_IBP: bounds of a consumer ReLU (or NULL)
  float* relu_hi;
  const float* addend;         // [opos][N] or NULL, added to acc before the epilogue
  const float* lo;             // (unused by the GEMM epilogues; kept for descriptors)
  const float* hi;
  const float4* coef;          // E_RELAX / E_ADJOINT: relaxation of the target at [b-pos][N]:
                               // {a (adaptive lower slope), s, t, column}: the int bits of w are
                               // -1 for a stable neuron, else its compact column (0 if not compact)
  const float* bias;           // per output channel (E_STORE / E_RELAX / E_IBP)
  int bias_c;                  // channels of the bias: index = n % bias_c (0: index = n)
  const float* alpha;          // E_RELAX: per [opos][N] lower slope of unstable neurons, or NULL
  float* psi_out;              // E_RELAX: store the pre-relaxation value v, or NULL
  // compact alpha (E_RELAX / E_ADJOINT): alpha, psi_out / psi_in and the Adam
  // state hold only unstable neurons, row r at r * acols + (column in coef.w);
  // aidx (the column map the coefficients were built from) non-NULL selects
  // this layout, else the [opos][N] layout
  const int* aidx;
  int acols;
  const float* center;         // E_CONCRETIZE: centre/radius of the domain box at [b-pos][N]
  const float* radius;         // NULL -> eps
  float* part;                 // row partials [M][part_ld] (column = N-tile index; gather:
                               // row index (Y*gw + X)*rows + row)
  int part_ld;
  int ksplit;                  // E_IBP / E_ADJOINT: > 1 splits K into slices; slice s writes its raw
                               // products to out (and out2) + s*M*N, reduced by
                               // launch_ibp_splitk_finish / launch_adjoint_finish
  // ---- E_ADJOINT (alpha-CROWN step): per [opos][N] of the ReLU after this node
  const float* psi_in;         // pre-relaxation product kept by the evaluation
  float* alpha_rw;             // lower slopes, updated in place
  float* adam_m;
  float* adam_v;
  int do_update;               // 0: gradient pass without the Adam update
  float lr, beta1, beta2, bc1, bc2, adam_eps;  // bc = 1 / (1 - beta^t)
  float* gz_out;               // or NULL: the adjoint over z (after its bias) at [opos][N]
};

// A one-tap, one-position descriptor is a plain GEMM (row-major m); anything
// else is a gather GEMM (position-major m).  Footprint rows are always a gather
// GEMM (their epilogue maps each row's window cells to pixels, even on 1 x 1
// windows).
inline bool gemm_is_dense(const GemmDesc& d) {
  return !d.patch && d.gh == 1 && d.gw == 1 && d.hs == 1 && d.ws == 1 && d.ntaps == 1 && d.cs == d.K && d.tap_dy[0] == 0 &&
         d.tap_dx[0] == 0 && d.tap_w[0] == 0 && d.ho == 1 && d.wo == 1;
}

// Launch the implicit GEMM; returns hipSuccess or the launch error.
hipError_t launch_gemm(const GemmDesc& d, hipStream_t st);

// Up to four gather GEMMs of one tile shape and epilogue as one grid (the
// output-parity classes of a strided transposed convolution).
constexpr int MAX_GEMM_MULTI = 4;
struct GemmMulti {
  GemmDesc d[MAX_GEMM_MULTI];
  int n;
  int first[MAX_GEMM_MULTI + 1];  // first workgroup slot (index / 8) of each descriptor's tiles
};
// Launch descriptors ds[0..n) (finalised here, taken longest reduction first) as
// one grid.  hipErrorNotSupported: they do not share a tile shape, epilogue
// variant or fast path (launch them one by one); nothing is launched then.
hipError_t launch_gemm_multi(const GemmDesc* ds, int n, hipStream_t st);
// Number of N-tiles launch_gemm uses for this descriptor (= partial columns).
int gemm_ntiles(const GemmDesc& d);

// rowacc[r] (+)= sum over z < Z, p < P, s < S of part[((z*rows + r)*P + p)*ld + s]
// (pos_major: part[((z*P + p)*rows + r)*ld + s])
hipError_t launch_rows_reduce(const float* part, int Z, int rows, int P, int S, int ld,
                              float* rowacc, int accumulate, int pos_major, hipStream_t st);

// Write the final outputs from row accumulators.  rows per batch element = 2R:
// lb[b*R + i] = acc[b*2R + i], ub[b*R + i] = -acc[b*2R + R + i]  (NULL skips);
// intersect: lb = max(lb, new), ub = min(ub, new) with the values already there
hipError_t launch_finish(const float* rowacc, int batch, int R, float* lb, float* ub,
                         float* best, hipStream_t st, int intersect = 0);
// Lower-only rows (R per batch element): lb[i] = acc[i], best[i] = max(best[i], acc[i])
// (best[i] = acc[i] when init).
hipError_t launch_finish_lower(const float* rowacc, long long n, float* lb, float* best, int init, hipStream_t st);

// Spec rows: lam[b][r][:] = +C[b][r][:] for r < m and -C[b][r-m][:] for r >= m;
// rowacc[b*2m + r] = lam[b][r][:] . bias (bias may be NULL; per channel: index j % bias_c).
hipError_t launch_spec_init(const float* C, int batch, int m, int n, const float* bias, int bias_c,
                            float* lam, float* rowacc, int rows_sign_split, hipStream_t st);

// Identity rows through a Linear node followed (backwards) by a ReLU relaxation:
// row (b, s, i), s in {+1,-1}: psi = s*W[i][:]; lam = relax(psi; lo/hi[b][:]);
// rowacc = s*bias_start[i] + sum_j lam_j bias_z[j] + min(psi_j,0) t_j
// bias_z is per channel of z: index j % bias_zc (z flattened from a [h][w][c] tensor).
// With sel (selected rows, [batch][n_out] neuron list, cnt [batch] valid entries): rows
// (b, s, u) for u < U are neuron sel[b][u] (zero rows when u >= cnt[b]), 2U per input.
hipError_t launch_identity_linear(const float* W, int n_out, int n_in, const float* bias_start,
                                  const float* lo, const float* hi, const float* bias_z, int bias_zc,
                                  int batch, float* lam, float* rowacc, hipStream_t st,
                                  const int* sel = nullptr, const int* cnt = nullptr, int U = 0);
// Selected identity rows written out over n neurons, with their bias terms in rowacc.
hipError_t launch_select_fill(int batch, int n, int U, const int* sel, const int* cnt, const float* bias, int bias_c,
                              float* lam, float* rowacc, hipStream_t st);
// sel[b][rank] = j for idx[b][j] = rank >= 0
hipError_t launch_rank_to_list(const int* idx, int batch, int n, int* sel, hipStream_t st);
// node bounds of the selected neurons from their 2U rows per input (optionally intersected)
hipError_t launch_finish_select(const float* acc, int batch, int U, int n, const int* sel, const int* cnt, float* lb,
                                float* ub, int intersect, hipStream_t st);

// Identity rows through a Conv node: rows (b, s, i) with i = (y*Wo + x)*Co + c over
// the conv output; psi over the conv input [Hi][Wi][Ci] is s*W[ky][kx][c][ci] on the
// kernel footprint (yy = y*stride + ky - pad) and 0 elsewhere.  mode E_STORE:
// out = psi (+ addend), row += psi . bias[ci] (if bias); E_RELAX: out = relax(psi +
// addend; lo/hi of the target [b][e]), row += out . bias[ci] + min(v,0) t;
// E_CONCRETIZE: row += v c - |v| r over the box (center/radius or lo/hi).
// W layout [kh][kw][Co][Ci].  rowacc[row] += row partial.
struct IdConv {
  const float* W;
  int Co, Ho, Wo, Ci, Hi, Wi, kh, kw, stride, pad;
  int mode;
  const float* addend;
  float* out;
  const float* lo;
  const float* hi;
  const float* bias;
  const float* center;
  const float* radius;
  float eps;
};
hipError_t launch_identity_conv(const IdConv& a, int batch, float* rowacc, hipStream_t st);

// Transposed conv from tap-expanded products: Q [rows][Ho*Wo][taps*Ci] holds
// Lambda . W[tap][:, ci] per output position; psi over the conv input is
// psi[row][y][x][ci] = sum over taps (ky, kx) with oy = (y + pad - ky) / stride
// integral and in range of Q[row][oy*Wo + ox][(ky*kw + kx)*Ci + ci].  The epilogue
// is E_STORE / E_RELAX / E_CONCRETIZE as for IdConv (plus psi_out); rowacc += row sum.
struct Col2Im {
  const float* Q;
  int Ho, Wo, Ci, Hi, Wi, kh, kw, stride, pad;
  int rows_per_b;
  int mode;
  const float* addend;
  float* out;
  float* psi_out;
  const float* lo;
  const float* hi;
  const float* bias;
  const float* center;
  const float* radius;
  float eps;
  // footprint windows (concretisation only): Hi x Wi is the row's window of an
  // img_h x img_w domain node; cell (y, x) of row p = (py, px) of a pgh x pgw
  // start node with pc channels is pixel (py*psy + poy + y, px*psx + pox + x)
  int patch, pc, pgh, pgw, psy, poy, psx, pox, img_h, img_w;
};
hipError_t launch_col2im(const Col2Im& a, int rows, float* rowacc, hipStream_t st);

// Lambda over the input of a conv with few input channels (the domain node),
// from Lambda over its output, concretised: L_in[row][y][x][ci] = sum over
// taps (ky, kx) with oy = (y + pad - ky) / stride and ox = (x + pad - kx) /
// stride exact and in range, and over output channels co, of
// L_out[row][oy][ox][co] W[ky][kx][co][ci] (+ addend); then
// rowacc[row] += sum L_in c - |L_in| r over the row's domain box.  Direct
// VALU kernel: a workgroup stages the output rows a band of input rows needs
// in LDS and each thread accumulates its pixels' Ci values (vb_kernels.hip).
struct ConvIn {
  const float* lam;     // [rows][Ho][Wo][Co]
  const float* W;       // [kh][kw][Co][Ci]
  int Co, Ho, Wo, Ci, Hi, Wi, kh, kw, stride, pad;
  int rows_per_b;
  const float* addend;  // [rows][Hi][Wi][Ci] or NULL
  float* psi_out;       // receives L_in, or NULL
  const float* center;  // [batch][Hi][Wi][Ci], or [batch][img_h][img_w][Ci] with patch
  const float* radius;  // or NULL -> eps
  float eps;
  // footprint windows (patch != 0; addend and psi_out NULL): Hi x Wi is the
  // row's window of an img_h x img_w domain node; cell (y, x) of row p =
  // (py, px) of a pgh x pgw start node with pc channels is pixel
  // (py*psy + poy + y, px*psx + pox + x)
  int patch, pc, pgh, pgw, psy, poy, psx, pox, img_h, img_w;
};
// Whether the direct kernel takes this shape (Ci <= 4, Co a multiple of 16 up to 64,
// at most 48 (tap, input channel) pairs, bands fit in LDS).
bool conv_input_fits(const ConvIn& a);
// part: rows * ceil(Hi / band rows) floats of scratch.
hipError_t launch_conv_input_concretize(const ConvIn& a, int rows, float* part, float* rowacc, hipStream_t st);
size_t conv_input_part_floats(const ConvIn& a, int rows);

// Identity rows over a node of C channels, each on its own 1 x 1 window:
// out [rows][C] with out[row][c'] = +-1 at c' = row's channel (rows_per_b = R).
hipError_t launch_patch_identity(int rows, int R, int C, float* out, hipStream_t st);
// The same rows written into a wh x ww window of C channels at cell (cy, cx):
// out [rows][wh][ww][C], sign at the row's channel of that cell, 0 elsewhere.
hipError_t launch_window_identity(int rows, int R, int C, int wh, int ww, int cy, int cx, float* out,
                                  hipStream_t st);
// A window [rows][sh][sw][C] copied into [rows][dh][dw][C] at cell offset (oy, ox),
// zeros elsewhere (the window must fit).
hipError_t launch_window_embed(const float* src, int rows, int C, int sh, int sw, int dh, int dw, int oy, int ox,
                               float* dst, hipStream_t st);
// The first back-substitution step of footprint identity rows through the start
// conv, relaxed at the ReLU below it, without a GEMM over the one-hot rows: row
// (b, sign, pixel p, channel c) gets sign * W[Y][X][c][:] on window cell (Y, X),
// relaxed with the coefficients of the cell's pixel of the ReLU input (zero
// outside the image); rowacc[row] += the row's bias and relaxation terms.
struct PatchIdRelax {
  const float* W;       // [kh][kw][Co][Ci] of the start conv
  int Co, Ci, kh, kw;   // start channels, channels of the node below, kernel
  int R;                // rows per input: 2 * pgh * pgw * Co
  int pgh, pgw;         // start node grid
  int psy, poy, psx, pox;  // window cell (Y, X) of pixel (py, px): (py*psy + poy + Y, px*psx + pox + X)
  int img_h, img_w;     // the node below
  const float4* coef;   // [b][img_h][img_w][Ci] relaxation coefficients
  const float* bias;    // per channel of the node below, or NULL
  float* out;           // [rows][kh][kw][Ci]
};
// Whether the kernel takes the shape.
bool patch_id_relax_fits(const PatchIdRelax& a);
hipError_t launch_patch_id_relax(const PatchIdRelax& a, int rows, float* rowacc, hipStream_t st);

// rowacc[b*2n + r] = s * bias[i % bias_c] for identity rows (s = +1 for r < n, -1 after; i = r mod n)
hipError_t launch_identity_bias(int batch, int n, const float* bias, int bias_c, float* rowacc, hipStream_t st);

// Identity rows materialised as a dense matrix: rows (b, s, i) over n, +-1 on the diagonal.
hipError_t launch_identity_fill(int batch, int n, float* lam, hipStream_t st);

// Standalone relaxation of lam over a ReLU with input bounds lo/hi [b][P*N]:
// src is [rows][P*N] (or [rows][N] broadcast over P positions with scale, for GAP);
// out = relax(src + addend); rowacc[r] += sum out.bias_z + min(v,0) t
// alpha / psi_out: [rows][P*N], or compact ([rows][acols] at column aidx[b][P*N]) if aidx != NULL.
hipError_t launch_relax(const float* src, int src_broadcast, float scale, const float* addend,
                        int rows, int rows_per_b, int P, int N, const float* lo, const float* hi,
                        const float* bias_z, const float* alpha, float* psi_out, const int* aidx, int acols,
                        float* out, float* rowacc, hipStream_t st);

// dst[i] = a[i] + b[i] (b may be NULL: copy), i < n
hipError_t launch_add(const float* a, const float* b, float scale_b, float* dst, long long n,
                      hipStream_t st);

// Broadcast lam over GAP: dst[r][p][c] = src[r][c] * scale (+ addend)
hipError_t launch_gap_expand(const float* src, int rows, int P, int C, float scale,
                             const float* addend, float* dst, hipStream_t st);

// Standalone concretisation: rowacc[r] (+)= sum_j A[r][j] c - |A[r][j]| rad
// with c/rad at [r/rows_per_b][j] (center NULL -> from lo/hi box; radius NULL -> eps)
hipError_t launch_concretize_rows(const float* A, int rows, int n, int rows_per_b,
                                  const float* center, const float* radius, float eps,
                                  const float* lo, const float* hi, const float* bias,
                                  float* lb, float* ub, float* rowacc, hipStream_t st);

// IBP elementwise nodes on [batch][n]: op 0 relu clamp, 1 add
hipError_t launch_ibp_eltwise(int op, const float* lo0, const float* hi0, const float* lo1,
                              const float* hi1, float* lo, float* hi, long long n, hipStream_t st);
// IBP GAP: lo/hi [b][c] = mean over P positions of [b][p][c]
hipError_t launch_ibp_gap(const float* lo_in, const float* hi_in, int batch, int P, int C,
                          float* lo, float* hi, hipStream_t st);

// dst[b][c][r] = src[b][r][c] for b < batch (weight layout changes)
hipError_t launch_transpose(const float* src, int batch, int R, int C, float* dst, hipStream_t st);

// alpha-CROWN set-up: alpha = adaptive lower slope of each neuron (1 if u >= -l
// else 0 when unstable; 1 active; 0 inactive) for every one of `rows_per_b`
// spec rows of each batch element; m = v = 0.  Bounds lo/hi [batch][n].
// With aidx != NULL the state is compact: [batch*rows_per_b][acols], neuron j of
// batch element b at column aidx[b][j] (unstable neurons only; -1 elsewhere).
hipError_t launch_alpha_init(const float* lo, const float* hi, int batch, int rows_per_b, long long n,
                             const int* aidx, int acols, float* alpha, float* adam_m, float* adam_v,
                             hipStream_t st);

// Compact alpha columns: for each batch element b, idx[b][j] = number of
// unstable neurons (l < 0 < u) before j in node order if j is unstable, else
// -1; count[b] = number of unstable neurons of b.  One workgroup per b.
hipError_t launch_alpha_layout(const float* lo, const float* hi, int batch, long long n, int* idx, int* count,
                               hipStream_t st);

// Adjoint at the input box: g[r][j] = c[b][j] - rad[b][j] * sign(psi[r][j]), b = r / rows_per_b
hipError_t launch_adj_domain(const float* psi, int rows, int n, int rows_per_b, const float* center,
                             const float* radius, float eps, float* g, hipStream_t st);

// Relaxation coefficients of n neurons from their bounds: {a, s, t, unstable}
// (inactive u <= 0: 0,0,0; active l >= 0: 1,1,0; unstable: adaptive a, s = u/(u-l), t = -s l)
// w holds the bits of an int: -1 for a stable neuron, else the neuron's column
// aidx[i] in a compact state layout (0 when aidx is NULL).
hipError_t launch_relax_coef(const float* lo, const float* hi, long long n, const int* aidx, float4* coef,
                             hipStream_t st);

// Box centre and radius of bounds: c = (lo+hi)/2, r = (hi-lo)/2, n elements
hipError_t launch_box_center_radius(const float* lo, const float* hi, long long n, float* c, float* r,
                                    hipStream_t st);

// lo = sum_s pc[s] + bias - sum_s pr[s], hi = ... + sum_s pr[s] over S slices of M*N
// (fixed order); relu bounds too if given.  bias per column n = e % N.
hipError_t launch_ibp_splitk_finish(const float* pc, const float* pr, int S, long long MN, int N,
                                    const float* bias, float* lo, float* hi, float* relu_lo,
                                    float* relu_hi, hipStream_t st);

// Fill with a constant
hipError_t launch_fill(float* p, float v, long long n, hipStream_t st);

// E_ADJOINT epilogue of a dense GEMM whose K was split: sums the S slices of
// part [S][M][N] and applies the ReLU adjoint and the Adam step (vb_kernels.hip).
struct AdjFinish {
  const float* part;
  int S, M, N, rows_per_b;
  const float* bias;
  const float4* coef;
  const float* psi_in;
  float* alpha_rw;
  float* adam_m;
  float* adam_v;
  const int* aidx;  // compact columns (see GemmDesc::aidx) or NULL
  int acols;
  int do_update;
  float lr, beta1, beta2, bc1, bc2, adam_eps;
  float* out;
  float* gz_out;    // or NULL: receives the adjoint over z (after z's bias), [M][N]
};
hipError_t launch_adjoint_finish(const AdjFinish& a, hipStream_t st);

// The alpha-CROWN adjoint through a conv over a few-channel input with the
// ReLU's adjoint epilogue, without an im2col image (vb_kernels.hip). The
// epilogue fields come from a: M = rows, N = Ho * Wo * Co (part, S unused).
struct ConvAdj {
  AdjFinish a;
  const float* g0;  // [rows][Hi][Wi][Ci] adjoint over the conv input
  const float* W;   // [kh][kw][Co][Ci]
  int Ci, Hi, Wi, Co, Ho, Wo, kh, kw, stride, pad;
};
// Whether the direct kernel takes this shape (Ci <= 4, Co a multiple of 16 up
// to 64, at most 36 (tap, input channel) pairs, a row's input image within 48 KB).
bool conv_adjoint_fits(const ConvAdj& c);
hipError_t launch_conv_adjoint_first(const ConvAdj& c, int rows, hipStream_t st);

// im2col of a [rows][H][W][C] tensor for a kh x kw conv (stride, pad) into
// [rows][Ho][Wo][Kp] with k = tap*C + c and zeros for k >= kh*kw*C; and the
// matching weights [tap][N][C] -> [N][Kp] (vb_kernels.hip).
hipError_t launch_im2col(const float* src, int rows, int H, int W, int C, int kh, int kw, int stride, int pad,
                         int Ho, int Wo, int Kp, float* dst, hipStream_t st);
hipError_t launch_pad_weights(const float* W, int taps, int N, int C, int Kp, float* dst, hipStream_t st);

// IBP through a Linear layer for a batch of at most 16 (vb_ibp_narrow.hip):
// weights streamed once, batch on the MFMA column dimension.
struct NarrowIbp {
  int batch, K, N;          // inputs, n_in, n_out
  int amode;                // A_IBP_BALL (A = centre, A2 = radius or NULL -> eps) or A_IBP_BOX (A = lo, A2 = hi)
  const float* A;
  const float* A2;
  float eps;
  const float* W;           // [N][K]
  const float* bias;        // [N] or NULL
  float* lo;                // [batch][N]
  float* hi;
  float* relu_lo;           // optional ReLU of the bounds
  float* relu_hi;
  float* pc;                // split-K partial sums [slices][batch][N] (centre, radius)
  float* pr;
  int kchunk;               // set by the launcher
  int slices;               // set by the launcher
  int packed;               // W is the packed copy (launch_pack_linear; K a multiple of 16)
};
bool ibp_narrow_fits(int batch, int K, const float* W, const float* A, const float* A2);
int ibp_narrow_slices(int N, int K);
hipError_t launch_ibp_narrow(NarrowIbp d, int S, hipStream_t st);
// The narrow kernel's packed weight layout: floats of the copy, and the copy.
size_t pack_linear_floats(int N, int K);
hipError_t launch_pack_linear(const float* W, int N, int K, float* dst, hipStream_t st);

// verified[b] = 1 iff every lb[b][i] > 0 (i < m); count[0] (if count) = number of verified inputs.
hipError_t launch_verify(const float* lb, int batch, int m, int* verified, int* count, hipStream_t st);

// beta-CROWN (branch-and-bound sub-domains):
// lo = max(lo, 0) where split > 0, hi = min(hi, 0) where split < 0 (n elements)
hipError_t launch_apply_splits(const float* split, long long n, float* lo, float* hi, hipStream_t st);
// lam[row][j] -= beta[row][j] * split[row / R][j]; rowacc[row] += the term's bias products
hipError_t launch_beta_apply(float* lam, int rows, int R, int n, const float* beta, const float* split,
                             const float* bias, int bias_c, float* rowacc, hipStream_t st);
// projected Adam ascent of beta (>= 0) with gradient -split * gz, on split neurons only
hipError_t launch_beta_adam(int rows, int R, int n, const float* gz, const float* split, float* beta, float* bm,
                            float* bv, float lr, float b1, float b2, float bc1, float bc2, float eps,
                            hipStream_t st);
// branching score [batch][n]: sum over the open rows (best <= 0) of max(-psi, 0) * t; -inf when stable
hipError_t launch_branch_score(const float* psi, const float* best, int batch, int R, int n, const float* lo,
                               const float* hi, float* score, hipStream_t st);
// dst[b][:] = src[:] for b < batch
hipError_t launch_broadcast(const float* src, long long n, int batch, float* dst, hipStream_t st);

// Fixed scratch of the allocation-free entry point (vb_scratch.hip): its size, and
// its address on the device of stream `st` (the null stream: the current device),
// looked up on the first call per device and cached.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(256) << 20;
hipError_t noalloc_scratch(hipStream_t st, void** ptr);

}  // namespace vb

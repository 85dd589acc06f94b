/* vb.h -- C ABI of the MI355X linear bound propagation library (libvbprop.so).
 *
 * Computes certified output bounds of ReLU networks over an input domain with
 * the bound-propagation algorithms named in "Scaling Neural Network
 * Verification with Tensor Parallelism and Fully Sharded Data Parallelism"
 * (Sec. 1, problem definition: a network, an input domain and a property; IBP,
 * CROWN and alpha-CROWN with their linear relaxation matrices A; Sec. 2.1:
 * relaxation slopes from intermediate bounds; Sec. 2.2: bound propagation
 * through convolutions; Sec. 3 / Sec. 4.3: per-neuron alpha slope tensors).
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    keeps no pointer after a call returns and allocates no device memory:
 *    scratch space comes from the caller's workspace (`ws`, `ws_bytes`), or,
 *    for vb_crown_noalloc, from a fixed scratch array in the library's code
 *    object.
 *  - Every call validates its arguments on the host first.  On an error
 *    nothing is enqueued and a negative status is returned; vb_last_error()
 *    then describes it.  Otherwise the work is enqueued on `stream` (a
 *    hipStream_t, passed as void*) and the call returns without synchronising.
 *    Asynchronous device faults surface at the caller's next synchronisation.
 *  - Results are deterministic: identical inputs give bitwise-identical
 *    outputs (all reductions run in a fixed order, no float atomics).
 *  - All data is float32.  Flat tensors are [batch][n].  Spatial tensors are
 *    channels-last: [batch][h][w][c].  A FLATTEN node reinterprets a
 *    [h][w][c] tensor as a vector in (h, w, c) order (no data movement).
 *  - Linear weights are [n_out][n_in] row-major.  Conv2d weights are
 *    [kh][kw][c_out][c_in] ("HWOI").  Biases are [n_out] / [c_out] or NULL.
 *  - The input domain is the L-inf box |x - x_center| <= r with
 *    r = x_radius[b][i] if x_radius is non-NULL, else the scalar eps.
 */
#ifndef VB_H
#define VB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vb_status;
#define VB_OK            0
#define VB_EINVAL       (-1)  /* null pointer, bad enum value, non-positive size */
#define VB_ESHAPE       (-2)  /* inconsistent graph or shapes                     */
#define VB_ENOMEM       (-3)  /* workspace too small (see vb_workspace_size)      */
#define VB_EDEVICE      (-4)  /* a HIP call or kernel launch failed               */
#define VB_EUNSUPPORTED (-5)  /* graph pattern this library does not handle       */

/* Node kinds.  Nodes are listed in topological order; node 0 is the input. */
#define VB_INPUT   0
#define VB_LINEAR  1
#define VB_CONV2D  2
#define VB_RELU    3
#define VB_ADD     4   /* elementwise sum of in0 and in1 (same shape)          */
#define VB_GAP     5   /* global average pool [h][w][c] -> [c]                  */
#define VB_FLATTEN 6   /* [h][w][c] -> [h*w*c]                                  */

typedef struct {
  int32_t op;                 /* VB_*                                            */
  int32_t in0, in1;           /* producer node indices, -1 if unused             */
  int32_t c, h, w;            /* output shape; flat nodes have h = w = 1         */
  int32_t kh, kw, stride, pad;/* conv2d only (zero padding, same in both dims)   */
  const float* weight;        /* device, borrowed for the call                   */
  const float* bias;          /* device or NULL                                  */
  const float* weight_packed; /* LINEAR: NULL, or the copy of weight that        */
                              /* vb_pack_linear wrote (device, 16-byte aligned,  */
                              /* borrowed for the call); vb_ibp then reads it    */
                              /* instead of weight for small batches            */
} vb_node;

typedef struct {
  int32_t n_nodes;
  const vb_node* nodes;       /* host array, borrowed for the call               */
} vb_graph;

/* Intermediate-bound methods for vb_crown. */
#define VB_METHOD_IBP    0   /* IBP bounds feed every ReLU relaxation             */
#define VB_METHOD_CROWN  1   /* CROWN bounds for every ReLU input (IBP where the  */
                             /* input is one affine step from the domain)         */
#define VB_METHOD_HYBRID 2   /* IBP up to node region_start, CROWN after it with  */
                             /* region_start's IBP box as the domain              */
#define VB_INTERSECT_IBP 16  /* flag for CROWN / HYBRID: each CROWN intermediate  */
                             /* bound is intersected with the node's IBP bound    */
                             /* (l = max, u = min) before later layers use it     */
#define VB_UNSTABLE_ONLY 64  /* flag for CROWN / HYBRID: rows only for the neurons */
                             /* of a Linear ReLU input that its IBP bounds leave  */
                             /* unstable (l < 0 < u); the others keep their IBP   */
                             /* bounds (their relaxation is already exact).  The  */
                             /* neuron lists are built on the device; launches    */
                             /* cover every neuron and the work of the stable     */
                             /* ones is skipped by whole workgroups (no host      */
                             /* synchronisation)                                  */
#define VB_ALPHA_ROWS    32  /* flag for vb_workspace_size: also enough for       */
                             /* vb_alpha_step_rows on the identity rows of every  */
                             /* ReLU input (alpha-CROWN intermediate bounds)      */

/* Thread-local description of the last error on this thread. */
const char* vb_last_error(void);

/* Bytes of workspace that lets every call below run on the whole batch at once
 * for this graph, batch size and spec count m.  A smaller workspace is accepted
 * as long as one batch element fits: the library then processes the batch in
 * chunks (same results). */
vb_status vb_workspace_size(const vb_graph* g, int32_t batch, int32_t m, int32_t method,
                            int32_t region_start, size_t* bytes);

/* Weight layout for IBP over wide Linear layers (Sec. 1 of the page: a hidden
 * layer of 262 144 neurons, whose weights IBP reads once per call).  For a
 * batch of at most 16, vb_ibp streams each Linear node's weights once through
 * the matrix cores; with a packed copy its load instructions read 1 KB of
 * contiguous memory each instead of 64-byte pieces of 16 rows.  The copy holds
 * the same numbers as weight ([n_out][n_in], n_in a multiple of 16) in blocks
 * of 16 rows x 16 columns, rows past n_out zero: vb_pack_linear_bytes gives its
 * size; vb_pack_linear writes it (enqueued on stream) into dst, which the
 * caller owns and passes as vb_node.weight_packed.  The copy is a snapshot:
 * pack again after changing the weights.  VB_EINVAL if n_in % 16 != 0, a size
 * is not positive, a pointer is NULL or dst is not 16-byte aligned; VB_ENOMEM
 * if dst_bytes is smaller than the size. */
vb_status vb_pack_linear_bytes(int32_t n_out, int32_t n_in, size_t* bytes);
vb_status vb_pack_linear(const float* weight, int32_t n_out, int32_t n_in, float* dst, size_t dst_bytes,
                         void* stream);

/* IBP (interval bound propagation, centre/radius form; Sec. 1 and Sec. 2.1 of
 * the page).  For every non-input node k with node_lo[k] != NULL, writes its
 * interval bounds [batch][size_k].  Affine nodes compute c' = W c + b and
 * r' = |W| r from (c, r) = ((l+u)/2, (u-l)/2) of their producer (the input
 * node hands over (x_center, radius) directly); ReLU clamps at 0; ADD sums;
 * GAP averages.  A node whose bounds another node reads (the source of an
 * affine node through flatten nodes, the input of a ReLU / ADD / GAP / FLATTEN,
 * the input of the last node when C is given) must have bounds storage
 * (node_lo[k] and node_hi[k] both non-NULL); a node nothing reads may have
 * none and is then skipped.  All of this is checked before anything is
 * enqueued.
 * If C != NULL (C: [batch][m][n_out] over the last node, which must be
 * LINEAR), also writes spec bounds spec_lo/spec_hi [batch][m] with C folded
 * into the last layer.  The workspace is optional without C: when it holds
 * the split-K partial sums (vb_workspace_size with m = 0), layers whose output
 * grid is small split their reduction over more workgroups; results are the
 * same up to the order of the fp32 sums. */
vb_status vb_ibp(const vb_graph* g, int32_t batch,
                 const float* x_center, const float* x_radius, float eps,
                 float* const* node_lo, float* const* node_hi,
                 const float* C, int32_t m, float* spec_lo, float* spec_hi,
                 void* ws, size_t ws_bytes, void* stream);

/* Compact storage of the per-neuron alpha state (Sec. 3 and Sec. 4.3 of the
 * page: the alpha slopes are the largest tensors of alpha-CROWN).  A slope is
 * only ever read for an unstable neuron (l < 0 < u), so the state of ReLU node
 * k can keep one column per unstable neuron: row r (batch element b = r / m)
 * of alpha[k], adam_m[k], adam_v[k] then has width[k] entries and neuron j of b
 * sits at column index[k][b][j] (-1 for a stable neuron, which has no entry).
 *   index: per node (host array of device pointers); for ReLU node k,
 *          [batch][size_k] int32, as written by vb_alpha_layout; others NULL.
 *   width: per node (host array); for ReLU node k the row length U_k >= the
 *          largest number of unstable neurons of any batch element.  A node
 *          with width 0 has no state: its alpha / Adam pointers may be NULL.
 * Columns past the count of a batch element are never read or written. */
typedef struct {
  const int32_t* const* index;
  const int32_t* width;
} vb_alpha_compact;

/* The compact alpha layout of the bounds node_lo / node_hi (of the ReLU
 * inputs): for every ReLU node k writes index[k] [batch][size_k] (device,
 * caller-owned) with the rank of each unstable neuron among the unstable
 * neurons of its batch element in node order, -1 for stable neurons, and
 * width[k] (host) = the largest count over the batch; width[k] = 0 for other
 * nodes.  ws must hold 4 * batch bytes.  This call SYNCHRONISES `stream` (the
 * widths are needed on the host to size the state). */
vb_status vb_alpha_layout(const vb_graph* g, int32_t batch, const float* const* node_lo,
                          const float* const* node_hi, int32_t* const* index, int32_t* width,
                          void* ws, size_t ws_bytes, void* stream);

/* One CROWN back-substitution (Sec. 1: the A matrices; Sec. 2.1: slopes from
 * intermediate bounds).  Rows over node `start`:
 *   C == NULL: identity rows; writes node bounds lb = l_start, ub = u_start,
 *              each [batch][size_start] (lb = lb(I), ub = -lb(-I));
 *   C != NULL: spec rows C [batch][m][size_start]; writes lb = lb(C) and
 *              ub = -lb(-C), each [batch][m].
 * The rows are pushed to `stop` through every node in between using the ReLU
 * relaxation of node_lo/node_hi of each ReLU input (adaptive lower slope, or
 * alpha), then concretised over the domain: the input box if stop == 0, else
 * the box [node_lo[stop], node_hi[stop]].  lb or ub may be NULL; with spec
 * rows and ub == NULL only the rows C are propagated (half the work).
 * alpha: NULL, or per node (entries of ReLU nodes between stop and start
 * non-NULL) the lower slopes [batch][m][size] used on unstable neurons
 * (Sec. 3 and Sec. 4.3: per-neuron alpha); needs C and ub == NULL (the slopes
 * bound one side: call again with -C for the upper bound).  compact: NULL, or
 * the compact layout of alpha (vb_alpha_compact; needs alpha).
 * If A_out != NULL, the linear bounds over `stop` are returned as well: the
 * rows are the 2R functions (+rows, then -rows, R = m or size_start; only the
 * R rows C when ub == NULL with spec rows) bounded
 * from below, row(x) >= A x + bias for x in the output of node `stop`, with
 * A_out [batch][2R][size_stop] (node layout: channels-last for conv nodes)
 * and bias_out [batch][2R] or NULL (beta: every bias met on the way, the
 * relaxation offsets; not the bias of `stop` itself).  lb/ub may then both be
 * NULL.  bias_out without A_out, or no output at all, is VB_EINVAL. */
vb_status vb_crown_backward(const vb_graph* g, int32_t batch, int32_t start, int32_t stop,
                            const float* C, int32_t m,
                            const float* const* node_lo, const float* const* node_hi,
                            const vb_alpha_compact* compact, const float* const* alpha,
                            const float* x_center, const float* x_radius, float eps,
                            float* lb, float* ub, float* A_out, float* bias_out,
                            void* ws, size_t ws_bytes, void* stream);

/* Concretisation of linear bounds over a box (Sec. 1: the A matrices).
 * A: [rows][n], bias: [rows] or NULL; row r belongs to batch element
 * r / rows_per_batch; center, radius: [batch][n] (radius NULL -> scalar eps).
 * lb[r] = A c - |A| r + bias, ub[r] = A c + |A| r + bias; either may be NULL. */
vb_status vb_concretize(int32_t rows, int32_t n, int32_t rows_per_batch,
                        const float* A, const float* bias,
                        const float* center, const float* radius, float eps,
                        float* lb, float* ub, void* stream);

/* alpha-CROWN set-up (Sec. 3 / Sec. 4.3 of the page: per-neuron alpha slope
 * tensors).  For every ReLU node k, alpha[k] [batch][m][size_k] receives the
 * adaptive CROWN lower slope of each neuron from the bounds of the ReLU's
 * input (1 if u >= -l else 0 for unstable neurons; 1 active; 0 inactive),
 * identical for the m spec rows of an input, and adam_m[k], adam_v[k] are
 * zeroed.  Entries for non-ReLU nodes are ignored (may be NULL), and so are
 * ReLU nodes whose alpha[k] is NULL (state that covers only some layers).  compact:
 * NULL (state [batch][m][size_k]), or the compact layout (vb_alpha_compact;
 * only the unstable neurons' columns are written). */
vb_status vb_alpha_init(const vb_graph* g, int32_t batch, int32_t m,
                        const float* const* node_lo, const float* const* node_hi,
                        const vb_alpha_compact* compact,
                        float* const* alpha, float* const* adam_m, float* const* adam_v, void* stream);

/* One alpha-CROWN step on the lower bounds of spec rows C [batch][m][n_out]
 * (Sec. 3 and Sec. 4.3 of the page: per-neuron alpha slope tensors).
 * alpha, adam_m, adam_v: per node, NULL except for ReLU nodes, each
 * [batch][m][size_k] (one lower slope per input, spec row and neuron; only the
 * unstable neurons' entries are read or changed), or in the compact layout
 * when compact != NULL (vb_alpha_compact).  Evaluates the CROWN lower
 * bound with these slopes into lb_out [batch][m] and folds it into best_lb
 * (elementwise max; at step == 1 best_lb is set to lb; best_lb may be NULL).
 * If step >= 1, then also takes one
 * bias-corrected Adam ascent step (step = Adam's 1-based t, learning rate lr,
 * beta1, beta2, adam_eps) on sum(lb) and clips alpha to [0, 1].  step == 0
 * only evaluates.  The domain is the input box (stop = node 0).  The graph
 * must be a chain (Linear/Conv, ReLU, Flatten; every affine node except the
 * last feeding one ReLU).  The gradient is the exact reverse-mode derivative of
 * sum(lb) (derivative branch psi >= 0 at psi = 0, sign(0) = 0 at the domain).
 * The workspace must hold the whole batch (see vb_workspace_size). */
vb_status vb_alpha_step(const vb_graph* g, int32_t batch, const float* C, int32_t m,
                        const float* const* node_lo, const float* const* node_hi,
                        const float* x_center, const float* x_radius, float eps,
                        const vb_alpha_compact* compact,
                        float* const* alpha, float* const* adam_m, float* const* adam_v,
                        int32_t step, float lr, float beta1, float beta2, float adam_eps,
                        float* lb_out, float* best_lb,
                        void* ws, size_t ws_bytes, void* stream);

/* Split constraints of branch-and-bound sub-domains (beta-CROWN; complete
 * verification, Sec. 2.2 and Sec. 4.3 of the page).  Each batch element is one
 * sub-domain of an input.  Per node (host arrays of device pointers, entries of
 * non-ReLU nodes ignored); for ReLU node k over input node z:
 *   split[k]:  [batch][size_z] +1 where the sub-domain requires z_j >= 0, -1
 *              where it requires z_j <= 0, 0 elsewhere; NULL: no constraint at k;
 *   beta[k]:   [batch][R][size_z] the rows' Lagrange multipliers (>= 0; only
 *              entries of split neurons are read), and beta_m[k], beta_v[k]
 *              their Adam moments (same shape).
 * With a beta state, every row bounds min C f(x) - sum_j beta_j split_j z_j(x)
 * over the relaxed network (a lower bound of C f on the sub-domain, where
 * split_j z_j >= 0), and a step raises beta with alpha by projected Adam
 * (beta >= 0; gradient -split * the adjoint over z).  The node bounds passed
 * with it must already be clamped to the splits (vb_apply_splits). */
typedef struct {
  const float* const* split;
  float* const* beta;
  float* const* beta_m;
  float* const* beta_v;
} vb_beta;

/* Clamp node bounds to split constraints, in place: for every ReLU node k with
 * split[k] != NULL, over its input node z: node_lo[z] = max(node_lo[z], 0)
 * where split > 0, node_hi[z] = min(node_hi[z], 0) where split < 0
 * ([batch][size_z] each). */
vb_status vb_apply_splits(const vb_graph* g, int32_t batch, const float* const* split, float* const* node_lo,
                          float* const* node_hi, void* stream);

/* alpha-CROWN step on rows over any Linear / Conv node `start` of a chain
 * network (the per-neuron alpha tensors of Sec. 3 and Sec. 4.3 of the page, on
 * intermediate layers as well as on the specification).  Rows:
 *   C != NULL: spec rows C [batch][m][size_start], lower bounds only, as in
 *              vb_alpha_step (which is this call with start = the last node);
 *              lb_out, best_lb [batch][m]; ub_out and best_ub must be NULL;
 *   C == NULL: the identity rows of `start`, +e_j (lower bound l_j) and -e_j
 *              (upper bound u_j) for every neuron j, R = 2 * size_start rows per
 *              input, each with its own slopes: alpha, adam_m, adam_v of every
 *              ReLU node below `start` are [batch][R][size_k] (compact:
 *              [batch][R][width_k]), rows 0..size-1 for +e_j then -e_j.
 *              lb_out / ub_out receive this evaluation's l and u [batch][size],
 *              best_lb / best_ub the best over the steps (step 1 sets them; later
 *              steps take the max of l and the min of u).  Any of the four may
 *              be NULL (not all).
 * beta: NULL, or the split constraints and multipliers of sub-domains
 * (vb_beta; dense alpha layout only; the workspace must then also hold
 * batch * R * (widest ReLU node below start) floats: vb_bab_workspace_size
 * covers it for spec rows).
 * Every row climbs its own bound: the objective is the sum of the rows' lower
 * bounds, whose gradient with respect to a row's slopes is that row's own.
 * The state of ReLU nodes at or above `start` is not used (may be NULL).  The
 * workspace must hold the whole batch (vb_workspace_size with VB_ALPHA_ROWS
 * covers the identity rows of every layer).  Other conventions as vb_alpha_step. */
vb_status vb_alpha_step_rows(const vb_graph* g, int32_t batch, int32_t start, const float* C, int32_t m,
                             const float* const* node_lo, const float* const* node_hi,
                             const float* x_center, const float* x_radius, float eps,
                             const vb_alpha_compact* compact, const vb_beta* beta,
                             float* const* alpha, float* const* adam_m, float* const* adam_v,
                             int32_t step, float lr, float beta1, float beta2, float adam_eps,
                             float* lb_out, float* best_lb, float* ub_out, float* best_ub,
                             void* ws, size_t ws_bytes, void* stream);

/* Branch and bound with beta-CROWN (complete verification of one input: the
 * page's Sec. 2.2 and Sec. 4.3 prove a ResNet this way).  Sub-domains are sets
 * of ReLU split constraints, bounded `batch` at a time as the batch elements of
 * one alpha-beta-CROWN run (intermediate bounds: the root's, clamped to the
 * splits; spec bounds: `steps` projected-Adam steps on alpha and beta from the
 * adaptive slopes and beta = 0, then one evaluation, best iterate kept).  The
 * queue is first-in first-out; a sub-domain is proved when every spec lower
 * bound is > 0, otherwise it is split on the unstable neuron with the largest
 * score sum over its unproved rows of max(-Psi_j, 0) * t_j (Psi over the ReLU
 * output, t = -u l / (u - l)), ties to the lowest (node, neuron), into the
 * sub-domains z_j >= 0 then z_j <= 0, appended to the queue.
 *   node_lo / node_hi: the root's bounds of every node [1][size] (device; e.g.
 *                      vb_crown with batch 1), not modified;
 *   C: [m][n_out] spec rows of the input; x_center [n0], x_radius [n0] or NULL;
 *   verdict (host): 1 when every sub-domain is proved, 0 when the search
 *                   stopped undecided (budget spent, or a sub-domain with no
 *                   unstable neuron left);
 *   domains (host): sub-domains bounded; root_lb (device [m] or NULL): the
 *                   root's best bound.
 * The graph must be a chain (as for vb_alpha_step).  This call SYNCHRONISES
 * `stream` twice per round (after copying the round's split constraints, and
 * when the bounds that decide the next sub-domains are read back); it
 * allocates nothing: the workspace must hold vb_bab_workspace_size bytes. */
typedef struct {
  int32_t steps;        /* Adam steps per sub-domain (then one evaluation) */
  float lr, beta1, beta2, adam_eps;
  int32_t batch;        /* sub-domains bounded together */
  int32_t max_domains;  /* sub-domains bounded before the search gives up */
} vb_bab_params;

vb_status vb_bab_workspace_size(const vb_graph* g, int32_t m, int32_t batch, size_t* bytes);
vb_status vb_bab(const vb_graph* g, const float* x_center, const float* x_radius, float eps,
                 const float* C, int32_t m, const float* const* node_lo, const float* const* node_hi,
                 const vb_bab_params* params, int32_t* verdict, int32_t* domains, float* root_lb,
                 void* ws, size_t ws_bytes, void* stream);

/* The whole bound computation for one batch: IBP for every node, then the
 * intermediate bounds of every ReLU input by `method`, overwriting node_lo /
 * node_hi of those nodes in topological order, then the spec bounds of C by
 * IBP (ibp_lb/ibp_ub, may be NULL) and by CROWN (lb/ub).  node_lo / node_hi
 * must be given for every non-input node. */
vb_status vb_crown(const vb_graph* g, int32_t batch,
                   const float* x_center, const float* x_radius, float eps,
                   int32_t method, int32_t region_start,
                   float* const* node_lo, float* const* node_hi,
                   const float* C, int32_t m,
                   float* ibp_lb, float* ibp_ub, float* lb, float* ub,
                   void* ws, size_t ws_bytes, void* stream);

/* The verdict (Sec. 1 of the page: the property must hold for every input of
 * the domain).  Spec rows are margins e_label - e_j, so the property of input
 * b is proved when every spec lower bound is positive: verified[b] = 1 if
 * lb[b][i] > 0 for all i < m (a NaN bound does not count), else 0.
 * lb: [batch][m] (device, e.g. the lb of vb_crown or the best_lb of the
 * alpha-CROWN steps); verified: [batch] int32 (device); n_verified: one int32
 * (device) receiving the number of verified inputs, or NULL. */
vb_status vb_verify(int32_t batch, int32_t m, const float* lb, int32_t* verified, int32_t* n_verified,
                    void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): vb_crown with
 * the library's own fixed device scratch in place of a caller workspace.  The
 * scratch is VB_NOALLOC_SCRATCH_BYTES (256 MiB) per GPU, held by every GPU the
 * library runs on until the process ends; it is found on the first call on a
 * device (make that first call outside any graph capture).  Nothing is
 * allocated.  A graph needing more than the scratch for one batch element is
 * rejected with VB_ENOMEM before anything is enqueued; a larger batch is
 * processed in chunks that fit (same results).  Every call on one GPU uses the
 * same scratch: calls that overlap on one GPU (different streams, or threads)
 * race and must be serialised by the caller.  The scratch keeps the last
 * call's contents; nothing in it is assumed to start at zero. */
#define VB_NOALLOC_SCRATCH_BYTES (256u << 20)
vb_status vb_crown_noalloc(const vb_graph* g, int32_t batch,
                           const float* x_center, const float* x_radius, float eps,
                           int32_t method, int32_t region_start,
                           float* const* node_lo, float* const* node_hi,
                           const float* C, int32_t m,
                           float* ibp_lb, float* ibp_ub, float* lb, float* ub, void* stream);

/* Measurement of the back-substitution GEMM (the dominant kernel), for
 * benchmarks only: these three calls keep process-wide state (a list of event
 * pairs), are not thread-safe, and add two event records per GEMM launch while
 * recording is on; no other entry point depends on them.
 * vb_profile_start() begins recording a pair of HIP events around every
 * back-substitution GEMM launch (relaxation, concretisation or store
 * epilogue), on the stream of that launch, together with its algorithmic FLOPs
 * (2 x rows x multiply-adds of the layer, without padding or tile waste).
 * vb_profile_stop() stops recording, waits for the recorded events and
 * returns the summed kernel time (ms), summed FLOPs and launch count.
 * vb_profile_record(i, ...) returns launch i of the last stopped recording:
 * its time (ms), algorithmic FLOPs and info[6] = {epilogue (0 store,
 * 1 relaxation, 2 concretisation), footprint windows (0/1), M, N, K, taps} of
 * the GEMM; VB_EINVAL when i is out of range. */
vb_status vb_profile_start(void);
vb_status vb_profile_stop(double* ms, double* flops, int64_t* launches);
vb_status vb_profile_record(int64_t i, double* ms, double* flops, int32_t* info);

#ifdef __cplusplus
}
#endif

#endif /* VB_H */

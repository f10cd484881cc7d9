/*
 * equitp — the E(3)-equivariant edge convolution of NequIP-style interatomic potentials as a
 * C-ABI library for AMD MI355X (gfx950).
 *
 * The operation (one message-passing convolution).  For every directed edge e = (s -> d) with
 * edge vector v_e (the library never looks at positions; callers typically use
 * v_e = pos[s] - pos[d], minimum image for periodic cells):
 *
 *   r = |v_e|, u = v_e / r
 *   Y_l(u)            real spherical harmonics, l = 0..L_sh, component normalisation
 *                     (sum_m Y_lm^2 = 2l + 1), m = -l..l, Y_1 = sqrt(3) (y, z, x)
 *   e_n(r)            = sqrt(2/r_c) sin(n pi r / r_c) / r * f(r / r_c), n = 1..n_radial,
 *                     f(t) = 1 - 28 t^6 + 48 t^7 - 21 t^8 for t < 1, else 0
 *   h                 = SiLU(e W1)          W1: [n_radial][hidden], no bias
 *   w                 = h W2                W2: [hidden][n_paths * C], column p * C + c
 *   out[d, l3, m3, c] += w[p, c] * sum_{m1, m2} C_p[m1, m2, m3] x[s, l1, m1, c] Y_l2[m2]
 *
 * for every path p = (l1, l2, l3) with l1 <= L_in, l2 <= L_sh, l3 <= L_out, |l1 - l2| <= l3 <=
 * l1 + l2 and l1 + l2 + l3 even, in lexicographic (l1, l2, l3) order; C_p is the unitary
 * real-basis Clebsch-Gordan block (Condon-Shortley phase).  This is the channelwise ("uvu")
 * tensor product with one radial weight per path and channel whose same-l3 paths are summed
 * inside the kernel (FlashCart, "Fast Cartesian Tensor Products for Equivariant Interatomic
 * Potentials", Fig. 3 caption), restricted to parity-coupled irreps (0e, 1o, 2e, 3o: "Fast and
 * Accurate Foundation Models for Equivariant Machine-Learned Interatomic Potentials", Sec. VII)
 * and computed in fp32 with fp32 sums (same page, Sec. II).  Messages are summed into receivers
 * with a receiver-sorted CSR segmented reduction (no atomics: results are bitwise reproducible).
 *
 * Layouts (all fp32 unless noted, row-major, channels innermost as in FlashCart Fig. D1):
 *   node tensors  [n_nodes][(L+1)^2][C], component index l*l + (m + l)
 *   vec           [n_edges][3]
 *   W1            [n_radial][hidden]
 *   W2            [hidden][n_paths * C]
 *   linear W      [L+1][C][C]   (W_l[u][v]: y[.., v] = sum_u feat[.., u] W_l[u][v])
 *
 * Ownership and streams.  Every array argument is a device pointer owned by the caller; the
 * library allocates no device memory in forward/backward (the caller passes a workspace).  Work is
 * enqueued asynchronously on the caller's stream (a hipStream_t passed as void*; NULL = default
 * stream); nothing synchronises.  Device faults surface at the caller's next synchronisation.
 * A handle holds host-side metadata only and may be shared by threads.
 *
 * Errors.  Every function returns an equitp_status; no exceptions cross the ABI.
 * Preconditions the library does not check (violations give undefined results): r > 0 for every
 * edge; indices in range; row_ptr non-decreasing with row_ptr[0] = 0 and row_ptr[n] = n_edges;
 * dst consistent with row_ptr.
 */
#ifndef EQUITP_H
#define EQUITP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EQUITP_OK = 0,
  EQUITP_INVALID_ARG = -1,         /* null/misaligned pointer, negative size, bad handle */
  EQUITP_IRREPS_PARSE = -2,        /* irreps string not of the form "Cx0e+Cx1o+..." */
  EQUITP_UNSUPPORTED = -3,         /* l > 3, mixed multiplicities (equitp_mixed_* takes those),
                                      parity != (-1)^l, C % 16 != 0, hidden not in {16, 64},
                                      n_radial != 8, L_in != L_sh != L_out */
  EQUITP_HIP_ERROR = -4,           /* a HIP runtime call or kernel launch failed */
  EQUITP_WORKSPACE_TOO_SMALL = -5  /* backward workspace smaller than equitp_backward_workspace */
} equitp_status;

typedef struct equitp_plan* equitp_t;

/* Graph, edges sorted by receiver.  All pointers are device pointers. */
typedef struct {
  int32_t n_nodes;
  int32_t n_edges;
  const int32_t* row_ptr;   /* [n_nodes + 1] receiver CSR: edges of d are row_ptr[d]..row_ptr[d+1]-1 */
  const int32_t* src;       /* [n_edges] sender of each edge */
  const int32_t* dst;       /* [n_edges] receiver of each edge (non-decreasing) */
  const int32_t* t_row_ptr; /* [n_nodes + 1] sender CSR over t_perm; needed only for grad_x */
  const int32_t* t_perm;    /* [n_edges] edge ids grouped by sender; needed only for grad_x */
  /* [n_edges] per-edge path subsets, or NULL (every edge computes every path).  Bit p of
   * path_mask[e] set: path p (W2's column order) is computed for edge e; a path that is off
   * contributes nothing to that edge's message, exactly as if its radial weights w[e, p, :] were
   * zero, in the forward and in every gradient (its dL/dw is zero too).  This is the adaptive
   * tensor-product computation of "BranchIP: Learning Adaptive Equivariant Computation for
   * Interatomic Potentials" (abstract) with the choice given as an input.  A path that no edge
   * of a 16-edge tile needs is skipped for the tile, so the saving follows from listing each
   * receiver's edges with similar masks next to each other (e.g. sorted by the number of paths
   * they keep).  Supported for fp32 operands, hidden = 64, l = 1..3 (EQUITP_UNSUPPORTED
   * otherwise). */
  const uint32_t* path_mask;
} equitp_graph;

/* Create a convolution.  irreps_in / irreps_out: "Cx0e+Cx1o+Cx2e[+Cx3o]" with one block per l
 * from 0 to L, uniform multiplicity C (a multiple of 16) and parity (-1)^l.  irreps_sh:
 * "1x0e+1x1o+..." (or "0e+1o+...") up to L_sh.  n_radial: number of Bessel functions.  Defaults:
 * hidden = 64, r_cut = 5.0 (change with equitp_set_radial).  On success *out is a new handle. */
int equitp_create(const char* irreps_in, const char* irreps_sh, const char* irreps_out,
                  int n_radial, equitp_t* out);

/* Radial MLP width and cutoff radius (Angstrom; edges with r >= r_cut carry zero messages). */
int equitp_set_radial(equitp_t h, int hidden, float r_cut);

/* Operand precision of the three radial-MLP contractions with W2 (the forward's w = h W2, the
 * backward's dL/dh = dL/dw W2^T and dL/dW2 = h^T dL/dw): 0 (default) fp32; 1 bf16 operands
 * (h, W2 and dL/dw rounded to nearest even) with fp32 accumulation, on the bf16 matrix cores.
 * The tensor product, the scatter sums and every other step stay fp32.  Mode 1 needs hidden = 64
 * and l >= 1 (EQUITP_UNSUPPORTED otherwise).  This is the mixed-precision training setting of
 * "High-performance training and inference for deep equivariant interatomic potentials" (the
 * dense contractions in reduced precision, reductions in fp32). */
int equitp_set_mlp_precision(equitp_t h, int bf16_operands);

/* Shape queries (any pointer may be NULL). */
int equitp_query(equitp_t h, int* n_paths, int* channels, int* f_in, int* f_sh, int* f_out,
                 int* w1_numel, int* w2_numel);

/* The (l1, l2, l3) of path p in W2's column order. */
int equitp_path(equitp_t h, int p, int* l1, int* l2, int* l3);

/* out [n_nodes][f_out][C] = the convolution (overwritten, receivers without edges get 0). */
int equitp_forward(equitp_t h, const equitp_graph* g, const float* vec, const float* x,
                   const float* W1, const float* W2, float* out, void* stream);

/* Workspace bytes needed by equitp_backward for this graph size. */
int equitp_backward_workspace(equitp_t h, int n_nodes, int n_edges, size_t* bytes);

/* Vector-Jacobian product for upstream gradient grad_out [n_nodes][f_out][C].  Outputs are
 * overwritten; any of them may be NULL to skip it: grad_vec [n_edges][3], grad_x
 * [n_nodes][f_in][C] (needs g->t_row_ptr and g->t_perm), grad_W1 [n_radial][hidden],
 * grad_W2 [hidden][n_paths * C].  workspace: device memory of at least
 * equitp_backward_workspace bytes, 256-byte aligned. */
int equitp_backward(equitp_t h, const equitp_graph* g, const float* vec, const float* x,
                    const float* W1, const float* W2, const float* grad_out, float* grad_vec,
                    float* grad_x, float* grad_W1, float* grad_W2, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Per-irrep channel-mixing linear on the matrix cores: for l = 0..lmax,
 * out[n, l*l + m, :] = feat[n, l*l + m, :] W_l (transpose_w = 0) or W_l^T (transpose_w = 1,
 * the data gradient of the former).  W: [lmax+1][C][C].  C must be a multiple of 16. */
int equitp_linear(int n_nodes, int lmax, int channels, const float* feat, const float* W,
                  int transpose_w, float* out, void* stream);

/* Build a CSR over edges grouped by an int32 key in [0, n_nodes): perm lists edge ids in
 * (key, edge id) order and row_ptr [n_nodes + 1] delimits each key's run.  Used for the sender
 * CSR (key = src).  Workspace from equitp_build_csr_workspace. */
int equitp_build_csr_workspace(int n_nodes, int n_edges, size_t* bytes);
int equitp_build_csr(int n_nodes, int n_edges, const int32_t* key, int32_t* row_ptr,
                     int32_t* perm, void* workspace, size_t workspace_bytes, void* stream);

/* The real-basis CG block of path (l1, l2, l3) as the kernels use it, copied densely into host
 * memory dense[(2l1+1)(2l2+1)(2l3+1)] (index (m1 * (2l2+1) + m2) * (2l3+1) + m3). */
int equitp_cg_block(int l1, int l2, int l3, float* dense);

/* Node-local product ladder with path-reduced products ("FlashCart: Fast Cartesian Tensor
 * Products for Equivariant Interatomic Potentials", Fig. 3(b): node-local tensor products by
 * correlation order, path-reduced with one scalar weight per path and channel; Fig. E1(b): the
 * same atomic basis A enters every product, and each product's output feeds the next one and
 * is added to the final sum).  Per node n and channel c, for correlation order nu:
 *
 *   B_1 = A
 *   B_s[l3 m3] = sum_p w[s-2][p][c] sum_{m1, m2} C_p[m1, m2, m3] B_{s-1}[l1 m1] A[l2 m2],  s = 2..nu
 *   out        = B_2 + B_3 + ... + B_nu
 *
 * over the paths p = (l1, l2, l3) with l1, l2, l3 <= lmax (triangle rule, l1 + l2 + l3 even,
 * lexicographic order; equitp_ladder_num_paths gives their number P).  The previous rung is the
 * first factor and A the second; A itself is not part of the sum.
 *
 * Layouts: A, out, grad_out, grad_A [n_nodes][(lmax+1)^2][channels] (node-tensor layout above);
 * w, grad_w [nu-1][P][channels].  Supported: lmax 0..3, nu 2..5, channels a positive multiple of
 * 16.  fp32 throughout.  forward overwrites out.  backward overwrites grad_A and grad_w for the
 * loss <grad_out, out>; either may be NULL to skip it; grad_w needs a workspace of at least
 * equitp_ladder_backward_workspace bytes (the size depends on the current device's CU count, so
 * query it on the device that runs the call).  n_nodes = 0 is a no-op apart from zeroing grad_w.
 * rungs (optional, training): [nu-2][n_nodes][(lmax+1)^2][channels] = B_2 .. B_{nu-1}.  The
 * forward writes them when rungs is not NULL (it is compute-bound, so the extra writes overlap
 * its arithmetic); a backward given the same rungs reads them instead of recomputing them.
 * NULL in either call: nothing kept / recomputed.  Unused for nu = 2.
 * Outputs must not alias inputs (EQUITP_INVALID_ARG).  Errors: EQUITP_UNSUPPORTED for an
 * unsupported lmax / nu / channel count, EQUITP_WORKSPACE_TOO_SMALL, EQUITP_HIP_ERROR for a failed
 * launch.  Results are bitwise reproducible (fixed-order reductions, no atomics). */
int equitp_ladder_num_paths(int lmax, int* n_paths);
int equitp_ladder_forward(int lmax, int nu, int n_nodes, int channels, const float* A,
                          const float* w, float* out, float* rungs, void* stream);
int equitp_ladder_backward_workspace(int lmax, int nu, int n_nodes, int channels, size_t* bytes);
int equitp_ladder_backward(int lmax, int nu, int n_nodes, int channels, const float* A,
                           const float* w, const float* rungs, const float* grad_out, float* grad_A,
                           float* grad_w, void* workspace, size_t workspace_bytes, void* stream);

/* Full product ladder ("FlashCart: Fast Cartesian Tensor Products for Equivariant Interatomic
 * Potentials", Fig. 3(b), dashed curves: the same node-local ladder with linear maps that mix
 * paths and channels between the products; Fig. E1(b): each product's outputs over the retained
 * coupling paths are compressed by a linear map W^(q) to d channels per rank).  Here d = channels
 * and every rank up to lmax is kept; the map of step s is one channels x channels matrix per
 * path, and the matrices of the paths into one l3 are summed:
 *
 *   T_p[n, m3, u]    = sum_{m1, m2} C_p[m1, m2, m3] B_{s-1}[n, l1 m1, u] A[n, l2 m2, u]
 *   B_s[n, l3 m3, v] = sum_{p -> l3} sum_u T_p[n, m3, u] W[s-2][p][u][v],   s = 2..nu
 *   out              = B_2 + ... + B_nu,   B_1 = A
 *
 * With W[s-2][p] = diag(w[s-2][p]) this is equitp_ladder_forward.  Paths and node-tensor layouts
 * as for the path-reduced ladder above; W, grad_W [nu-1][P][channels][channels] (row u, column v).
 * Supported: lmax 0..3, nu 2..5, channels 32, 64 or 128, n_nodes <= 2^26.  fp32 throughout (the
 * mixing runs on fp32 matrix cores).  Both calls need a workspace of at least
 * equitp_full_ladder_workspace bytes (backward = 0 for the forward, 1 for the backward); it holds
 * the path outputs of one step (n_nodes * sum_p (2 l3 + 1) * channels floats), the rungs when the
 * caller keeps none, and (backward) the next step's output gradient and dL/dW partials.  rungs:
 * as for the path-reduced ladder (the forward writes B_2 .. B_{nu-1} there when not NULL; a
 * backward given them reads them, else recomputes them).  saved (optional, training):
 * equitp_full_ladder_saved_floats floats, [nu-1][n_nodes * sum_p (2 l3 + 1)][channels] = every
 * step's path outputs T_p; a forward given it keeps them there (it has to write them anyway), and
 * a backward given the same buffer reads them for grad_W instead of computing them again.  288 GB
 * of HBM per GPU leave room: 0.8 GB at 4096 nodes, lmax 3, 128 channels, nu 5.  The forward overwrites out; the
 * backward overwrites grad_A and grad_W for the loss <grad_out, out>, either may be NULL.
 * n_nodes = 0 is a no-op apart from zeroing grad_W.  Outputs must not alias inputs
 * (EQUITP_INVALID_ARG); every tensor and the workspace must be 16-byte aligned
 * (EQUITP_INVALID_ARG).  Errors: EQUITP_UNSUPPORTED, EQUITP_WORKSPACE_TOO_SMALL,
 * EQUITP_HIP_ERROR.  Results are bitwise reproducible (dL/dW: partial maps per range of rows
 * summed per path in a fixed order; no atomics). */
int equitp_full_ladder_workspace(int lmax, int nu, int n_nodes, int channels, int backward,
                                 size_t* bytes);
int equitp_full_ladder_saved_floats(int lmax, int nu, int n_nodes, int channels, size_t* n);
int equitp_full_ladder_forward(int lmax, int nu, int n_nodes, int channels, const float* A,
                               const float* W, float* out, float* rungs, float* saved,
                               void* workspace, size_t workspace_bytes, void* stream);
int equitp_full_ladder_backward(int lmax, int nu, int n_nodes, int channels, const float* A,
                                const float* W, const float* rungs, const float* saved,
                                const float* grad_out, float* grad_A, float* grad_W,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Edge convolution with its own channel count per rotation order ("Fast and Accurate Foundation
 * Models for Equivariant MLIPs", Sec. III, Table 1: e.g. 128, 64, 32, 32 channels for l = 0..3
 * in the large NequIP model).  irreps_in / irreps_out: "128x0e+64x1o+32x2e+32x3o" — one block per l
 * from 0 to L (1..3), parity (-1)^l, each multiplicity a multiple of 32 up to 128; the spherical
 * harmonics go to L.  Per edge e = (s -> d), with r, Y and the radial MLP of equitp_create
 * (n_radial = 8 Bessel functions, hidden = 64 only):
 *
 *   w = SiLU(e(r) W1) W2                                   W2 [hidden][sum_p m_in[l1(p)]]
 *   M_p[d, m3, u] += w[e, p, u] sum_{m1,m2} C_p[m1,m2,m3] x[s, l1 m1, u] Y_l2[m2]    (u < m_in[l1])
 *   out[d, l3 m3, v] = sum_{p -> l3} sum_u M_p[d, m3, u] Wlin_p[u, v]              (v < m_out[l3])
 *
 * i.e. channelwise products per path (a path carries the m_in[l1] channels of its input rank),
 * receiver sums kept per path, then one channel-mixing linear map per path into the output rank.
 * Paths in the convolution's lexicographic order; W2's columns hold a block of m_in[l1] columns per
 * path; Wlin is the concatenation over paths of [m_in[l1]][m_out[l3]] row-major.  Mixed node tensors
 * (x, out, grad_out, grad_x) are [n_nodes][f] with f = sum_l (2l+1) m[l]: the blocks of l = 0, 1, ...
 * in order, block l holding 2l+1 rows of m[l] channels.  With every multiplicity equal and every
 * Wlin_p the identity this is equitp_forward.
 *
 * Computed from the uniform kernels: channel slices between consecutive distinct input
 * multiplicities, per slice masked convolutions keeping one path per output rank per launch, and the
 * maps on the fp32 matrix cores (equitp_mixed_query reports the slice and launch counts).  The graph
 * must not carry path_mask (EQUITP_INVALID_ARG).  x, W2, Wlin, out, saved and the gradients
 * other than grad_vec and grad_W1 must be 16-byte aligned, the workspace 256-byte aligned
 * (EQUITP_INVALID_ARG).  Workspace: at least equitp_mixed_workspace bytes
 * (backward = 0 / 1; depends on the current device for the backward).  The backward overwrites the
 * requested gradients (any may be NULL): grad_vec [n_edges][3], grad_x (needs g->t_row_ptr and
 * g->t_perm), grad_W1 [8][64], grad_W2, grad_Wlin for the loss <grad_out, out>.  saved
 * (optional, training): equitp_mixed_saved_floats floats; a forward given it keeps every path's
 * receiver sums there, and a backward given the same buffer reads them instead of recomputing
 * them for grad_Wlin (NULL: nothing kept / recomputed when grad_Wlin is wanted).  Results are
 * bitwise reproducible.  Errors as for equitp_create / equitp_backward. */
typedef struct equitp_mixed* equitp_mixed_t;
int equitp_mixed_create(const char* irreps_in, const char* irreps_out, int n_radial, int hidden,
                        float r_cut, equitp_mixed_t* out);
int equitp_mixed_query(equitp_mixed_t h, int* n_paths, int* f_in, int* f_out, int* w2_numel,
                       int* wlin_numel, int* n_slices, int* n_launches);
int equitp_mixed_workspace(equitp_mixed_t h, int n_nodes, int n_edges, int backward, size_t* bytes);
int equitp_mixed_saved_floats(equitp_mixed_t h, int n_nodes, size_t* n);
int equitp_mixed_forward(equitp_mixed_t h, const equitp_graph* g, const float* vec, const float* x,
                         const float* W1, const float* W2, const float* Wlin, float* out,
                         float* saved, void* workspace, size_t workspace_bytes, void* stream);
int equitp_mixed_backward(equitp_mixed_t h, const equitp_graph* g, const float* vec,
                          const float* x, const float* W1, const float* W2, const float* Wlin,
                          const float* saved, const float* grad_out, float* grad_vec,
                          float* grad_x, float* grad_W1, float* grad_W2, float* grad_Wlin,
                          void* workspace, size_t workspace_bytes, void* stream);
void equitp_mixed_destroy(equitp_mixed_t h);

void equitp_destroy(equitp_t h);
const char* equitp_status_string(int status);

/* Kernel timing (tracing).  While enabled, a pair of HIP events brackets every unit the library
 * launches (one kernel, or a fixed set such as the path-group kernels of one backward pass),
 * recorded on the stream the unit runs on; the events only time (no system-scope fence).
 * equitp_profile_get waits for the recorded events and returns, for the i-th unit name seen since
 * the last reset, the number of launches and their summed duration in milliseconds.  Not
 * thread-safe against concurrent launches from several host threads. */
int equitp_profile_enable(int on);
/* Restrict the timing to the units named in `names`, a comma-separated list of the names
 * equitp_profile_get reports (e.g. "bwd"); NULL or "" times every unit again.  Each recorded event
 * costs the stream a few microseconds, so a caller timing a sequence of many small launches can
 * bracket only the unit it studies.  The string is copied. */
int equitp_profile_only(const char* names);
int equitp_profile_reset(void);
int equitp_profile_count(void);
int equitp_profile_get(int i, const char** name, int* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* EQUITP_H */

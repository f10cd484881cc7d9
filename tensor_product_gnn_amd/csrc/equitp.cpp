// Host side of the equitp C ABI: irreps parsing, path enumeration, argument validation,
// workspace layout and the kernel sequence of forward and backward.
#include "../../include/equitp.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cctype>
#include <cstdint>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "cg_table.h"
#include "full_ladder.h"
#include "mixed.h"
#include "params.h"

struct equitp_plan {
  equitp::ConvShape shape;
  std::vector<int> path_l1, path_l2, path_l3;
};

namespace {

struct Block {
  int mul, l, parity;  // parity +1 even, -1 odd
};

// Parses "128x0e+128x1o" or "0e+1o" (multiplicity 1 when omitted).  Returns false on syntax error.
bool parse_irreps(const char* s, std::vector<Block>& out) {
  out.clear();
  if (s == nullptr) return false;
  std::string str;
  for (const char* c = s; *c; ++c)
    if (!std::isspace(static_cast<unsigned char>(*c))) str.push_back(*c);
  if (str.empty()) return false;
  size_t pos = 0;
  while (pos <= str.size()) {
    size_t end = str.find('+', pos);
    if (end == std::string::npos) end = str.size();
    const std::string tok = str.substr(pos, end - pos);
    if (tok.empty()) return false;
    Block b{1, 0, 1};
    size_t xp = tok.find('x');
    std::string lp = tok;
    if (xp != std::string::npos) {
      const std::string m = tok.substr(0, xp);
      if (m.empty() || m.size() > 9) return false;
      for (char c : m)
        if (!std::isdigit(static_cast<unsigned char>(c))) return false;
      b.mul = std::atoi(m.c_str());
      lp = tok.substr(xp + 1);
    }
    if (lp.size() < 2 || lp.size() > 3) return false;
    const char par = lp.back();
    const std::string ls = lp.substr(0, lp.size() - 1);
    for (char c : ls)
      if (!std::isdigit(static_cast<unsigned char>(c))) return false;
    b.l = std::atoi(ls.c_str());
    if (par == 'e') b.parity = 1;
    else if (par == 'o') b.parity = -1;
    else return false;
    out.push_back(b);
    if (end == str.size()) break;
    pos = end + 1;
  }
  return true;
}

// One block per l = 0..L in order, parity (-1)^l, uniform multiplicity.  Returns status.
int check_blocks(const std::vector<Block>& b, int* L, int* mul) {
  if (b.empty()) return EQUITP_IRREPS_PARSE;
  for (size_t i = 0; i < b.size(); ++i) {
    if (b[i].l != (int)i) return EQUITP_UNSUPPORTED;
    if (b[i].parity != ((b[i].l % 2) ? -1 : 1)) return EQUITP_UNSUPPORTED;
    if (b[i].mul != b[0].mul) return EQUITP_UNSUPPORTED;
  }
  *L = (int)b.size() - 1;
  *mul = b[0].mul;
  if (*L > 3) return EQUITP_UNSUPPORTED;
  return EQUITP_OK;
}

int n_cu_of_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

int feat(int L) { return (L + 1) * (L + 1); }

struct BwdLayout {
  size_t dvec, dw2, dw1, tiles, sort, sort_bytes, total;
  int wps, grid;
};

BwdLayout bwd_layout(const equitp::ConvShape& s, int n_edges, int n_cu) {
  BwdLayout b{};
  const size_t E = (size_t)(n_edges > 0 ? n_edges : 0);
  const int n_slices = s.C / 16;
  b.wps = equitp::bwd_wg_per_slice(s, n_edges, n_cu);
  b.grid = b.wps * n_slices;
  size_t off = 0;
  b.dvec = off;
  off += align256((size_t)n_slices * E * 3 * sizeof(float));
  b.dw2 = off;
  off += align256((size_t)b.wps * s.hidden * s.n_paths * s.C * sizeof(float));
  b.dw1 = off;
  off += align256((size_t)b.grid * s.n_radial * s.hidden * sizeof(float));
  // per-edge path subsets: the tile order of the backward and the sort's scratch
  b.tiles = off;
  off += align256((E + 15) / 16 * sizeof(int32_t));
  b.sort = off;
  b.sort_bytes = align256(equitp::tile_order_workspace_bytes((int)E));
  off += b.sort_bytes;
  b.total = off;
  return b;
}

int hip_status(hipError_t e) { return e == hipSuccess ? EQUITP_OK : EQUITP_HIP_ERROR; }

// ---------------------------------------------------------------------------------------------
// Kernel timing: events around each launch, on the launch's stream.
// ---------------------------------------------------------------------------------------------
struct ProfEntry {
  std::string name;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  int launches = 0;
  double total_ms = 0.0;
};
bool g_prof_on = false;
std::string g_prof_only;   // ",name1,name2," or empty: every unit
std::vector<ProfEntry> g_prof;
std::vector<hipEvent_t> g_ev_pool;

hipEvent_t prof_event() {
  if (!g_ev_pool.empty()) {
    hipEvent_t e = g_ev_pool.back();
    g_ev_pool.pop_back();
    return e;
  }
  // The events only time launches (read with hipEventElapsedTime once the caller has synchronised
  // the device), so they are created without the system-scope fence a default event performs at
  // every record: that fence writes back and invalidates the caches between launches, costs
  // several microseconds per event and slows the launch that follows.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// (The entry is kept by index: another scope may add entries and move the vector.)
struct ProfScope {
  int entry = -1;
  hipEvent_t a = nullptr, b = nullptr;
  hipStream_t st;
  ProfScope(const char* name, hipStream_t stream) : st(stream) {
    if (!g_prof_on) return;
    if (!g_prof_only.empty() && g_prof_only.find("," + std::string(name) + ",") == std::string::npos)
      return;
    for (size_t i = 0; i < g_prof.size(); ++i)
      if (g_prof[i].name == name) entry = (int)i;
    if (entry < 0) {
      g_prof.push_back(ProfEntry{name, {}, 0, 0.0});
      entry = (int)g_prof.size() - 1;
    }
    a = prof_event();
    b = prof_event();
    if (a && b) hipEventRecord(a, st);
  }
  ~ProfScope() {
    if (entry >= 0 && entry < (int)g_prof.size() && a && b) {
      hipEventRecord(b, st);
      g_prof[entry].ev.push_back({a, b});
    }
  }
};

// Product-ladder launch layout; returns a status.
int ladder_layout(int lmax, int nu, int n_nodes, int channels, int n_cu, equitp::LadderParams* p) {
  if (n_nodes < 0 || channels <= 0) return EQUITP_INVALID_ARG;
  if (lmax < 0 || lmax > 3 || nu < 2 || nu > 5 || channels % 16 != 0) return EQUITP_UNSUPPORTED;
  *p = equitp::LadderParams{};
  p->n_nodes = n_nodes;
  p->C = channels;
  p->cw = channels % 64 == 0 ? 64 : (channels % 32 == 0 ? 32 : 16);
  p->n_groups = channels / p->cw;
  const int npw = 64 / p->cw;
  const long long n_ng = ((long long)n_nodes + npw - 1) / npw;
  if (n_ng * p->n_groups > (1LL << 30)) return EQUITP_UNSUPPORTED;
  p->n_tasks = (int)(n_ng * p->n_groups);
  // backward: three work-groups per CU (47 KB of LDS and at most 168 VGPRs each at lmax 3, nu 5)
  const int target = 3 * (n_cu > 0 ? n_cu : 256) / p->n_groups;
  p->blocks_per_group = (int)std::max<long long>(1, std::min<long long>(n_ng, std::max(1, target)));
  return EQUITP_OK;
}

// dL/dw partial rows [blocks_per_group][nu-1][P][C], then the reduction's intermediate rows
size_t ladder_part_bytes(const equitp::LadderParams& p, int lmax, int nu) {
  return align256((size_t)p.blocks_per_group * (nu - 1) * equitp::ladder_num_paths(lmax) * p.C *
                  sizeof(float));
}
size_t ladder_workspace_bytes(const equitp::LadderParams& p, int lmax, int nu) {
  return ladder_part_bytes(p, lmax, nu) + (size_t)equitp::ladder_reduce_split() * (nu - 1) *
                                              equitp::ladder_num_paths(lmax) * p.C * sizeof(float);
}

// Per-edge path subsets: supported for fp32 operands, hidden width 64, l = 1..3 (at most 32 paths).
int mask_status(const equitp::ConvShape& s, const equitp_graph* g) {
  if (g->path_mask == nullptr) return EQUITP_OK;
  if (s.mlp_bf16 || s.hidden != 64 || s.L_in < 1 || s.L_in > 3 || s.n_paths > 32)
    return EQUITP_UNSUPPORTED;
  return EQUITP_OK;
}

bool graph_ok(const equitp_graph* g) {
  if (g == nullptr || g->n_nodes < 0 || g->n_edges < 0) return false;
  if (g->row_ptr == nullptr && g->n_nodes > 0) return false;
  if (g->n_edges > 0 && (g->src == nullptr || g->dst == nullptr)) return false;
  return true;
}

}  // namespace

extern "C" {

int equitp_create(const char* irreps_in, const char* irreps_sh, const char* irreps_out,
                  int n_radial, equitp_t* out) {
  if (out == nullptr) return EQUITP_INVALID_ARG;
  *out = nullptr;
  std::vector<Block> bi, bs, bo;
  if (!parse_irreps(irreps_in, bi) || !parse_irreps(irreps_sh, bs) || !parse_irreps(irreps_out, bo))
    return EQUITP_IRREPS_PARSE;
  int L_in, C_in, L_sh, m_sh, L_out, C_out;
  int st;
  if ((st = check_blocks(bi, &L_in, &C_in)) != EQUITP_OK) return st;
  if ((st = check_blocks(bs, &L_sh, &m_sh)) != EQUITP_OK) return st;
  if ((st = check_blocks(bo, &L_out, &C_out)) != EQUITP_OK) return st;
  if (m_sh != 1) return EQUITP_UNSUPPORTED;
  if (C_in != C_out || C_in <= 0 || C_in % 16 != 0) return EQUITP_UNSUPPORTED;
  if (n_radial <= 0) return EQUITP_INVALID_ARG;
  if (n_radial != 8) return EQUITP_UNSUPPORTED;
  if (L_in != L_sh || L_in != L_out) return EQUITP_UNSUPPORTED;
  equitp_plan* h = new (std::nothrow) equitp_plan();
  if (h == nullptr) return EQUITP_INVALID_ARG;
  h->shape.L_in = L_in;
  h->shape.L_sh = L_sh;
  h->shape.L_out = L_out;
  h->shape.C = C_in;
  h->shape.n_radial = n_radial;
  h->shape.hidden = 64;
  h->shape.r_cut = 5.0f;
  h->shape.mlp_bf16 = 0;
  // paths in lexicographic (l1, l2, l3) order: triangle rule, l1 + l2 + l3 even
  for (int l1 = 0; l1 <= L_in; ++l1)
    for (int l2 = 0; l2 <= L_sh; ++l2)
      for (int l3 = 0; l3 <= L_out; ++l3)
        if (l3 >= std::abs(l1 - l2) && l3 <= l1 + l2 && (l1 + l2 + l3) % 2 == 0) {
          h->path_l1.push_back(l1);
          h->path_l2.push_back(l2);
          h->path_l3.push_back(l3);
        }
  h->shape.n_paths = (int)h->path_l1.size();
  *out = h;
  return EQUITP_OK;
}

int equitp_set_radial(equitp_t h, int hidden, float r_cut) {
  if (h == nullptr || !(r_cut > 0.0f)) return EQUITP_INVALID_ARG;
  if (hidden != 16 && hidden != 64) return EQUITP_UNSUPPORTED;
  if (h->shape.mlp_bf16 && hidden != 64) return EQUITP_UNSUPPORTED;
  h->shape.hidden = hidden;
  h->shape.r_cut = r_cut;
  return EQUITP_OK;
}

int equitp_set_mlp_precision(equitp_t h, int bf16_operands) {
  if (h == nullptr || (bf16_operands != 0 && bf16_operands != 1)) return EQUITP_INVALID_ARG;
  if (bf16_operands && (h->shape.hidden != 64 || h->shape.L_in < 1)) return EQUITP_UNSUPPORTED;
  h->shape.mlp_bf16 = bf16_operands;
  return EQUITP_OK;
}

int equitp_query(equitp_t h, int* n_paths, int* channels, int* f_in, int* f_sh, int* f_out,
                 int* w1_numel, int* w2_numel) {
  if (h == nullptr) return EQUITP_INVALID_ARG;
  const equitp::ConvShape& s = h->shape;
  if (n_paths) *n_paths = s.n_paths;
  if (channels) *channels = s.C;
  if (f_in) *f_in = feat(s.L_in);
  if (f_sh) *f_sh = feat(s.L_sh);
  if (f_out) *f_out = feat(s.L_out);
  if (w1_numel) *w1_numel = s.n_radial * s.hidden;
  if (w2_numel) *w2_numel = s.hidden * s.n_paths * s.C;
  return EQUITP_OK;
}

int equitp_path(equitp_t h, int p, int* l1, int* l2, int* l3) {
  if (h == nullptr || p < 0 || p >= h->shape.n_paths) return EQUITP_INVALID_ARG;
  if (l1) *l1 = h->path_l1[p];
  if (l2) *l2 = h->path_l2[p];
  if (l3) *l3 = h->path_l3[p];
  return EQUITP_OK;
}

int equitp_forward(equitp_t h, const equitp_graph* g, const float* vec, const float* x,
                   const float* W1, const float* W2, float* out, void* stream) {
  if (h == nullptr || !graph_ok(g)) return EQUITP_INVALID_ARG;
  if (g->n_nodes == 0) return EQUITP_OK;
  if (out == nullptr || W1 == nullptr || W2 == nullptr || x == nullptr) return EQUITP_INVALID_ARG;
  if (g->n_edges > 0 && vec == nullptr) return EQUITP_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out) || !aligned4(W1) || !aligned4(W2)) return EQUITP_INVALID_ARG;
  if (int ms = mask_status(h->shape, g)) return ms;
  const int n_cu = n_cu_of_current_device();
  if (n_cu <= 0) return EQUITP_HIP_ERROR;
  equitp::SegParams p{};
  p.n_seg = g->n_nodes;
  p.C = h->shape.C;
  p.n_slices = h->shape.C / 16;
  p.seg_ptr = g->row_ptr;
  p.seg_edge = nullptr;
  p.gather = g->src;
  p.vec = vec;
  p.feat = x;
  p.W1 = W1;
  p.W2 = W2;
  p.out = out;
  p.inv_r_cut = 1.0f / h->shape.r_cut;
  p.radial_pref = std::sqrt(2.0f / h->shape.r_cut);
  p.path_mask = g->path_mask;
  ProfScope ps("seg_fwd", (hipStream_t)stream);
  return hip_status(p.path_mask ? equitp::launch_seg_conv_masked(h->shape, false, p, n_cu,
                                                                 (hipStream_t)stream)
                                : equitp::launch_seg_conv(h->shape, false, p, n_cu, (hipStream_t)stream));
}

int equitp_backward_workspace(equitp_t h, int n_nodes, int n_edges, size_t* bytes) {
  if (h == nullptr || bytes == nullptr || n_nodes < 0 || n_edges < 0) return EQUITP_INVALID_ARG;
  int n_cu = n_cu_of_current_device();
  if (n_cu <= 0) n_cu = 256;
  *bytes = bwd_layout(h->shape, n_edges, n_cu).total;
  return EQUITP_OK;
}

namespace {

// equitp_backward, plus settings for callers whose masks are the same on every edge: only the
// path groups in `groups` run (bit g = group g; the other groups' paths must be off), and the
// tile order is the identity (sorting equal tiles gains nothing); with tiles_ready the caller
// guarantees that the workspace already holds that identity order for this edge count (an earlier
// call with the same workspace wrote it), so it is not written again.
int backward_impl(equitp_t h, const equitp_graph* g, const float* vec, const float* x,
                  const float* W1, const float* W2, const float* grad_out, float* grad_vec,
                  float* grad_x, float* grad_W1, float* grad_W2, void* workspace,
                  size_t workspace_bytes, void* stream, unsigned groups, bool uniform_mask,
                  bool tiles_ready = false) {
  if (h == nullptr || !graph_ok(g)) return EQUITP_INVALID_ARG;
  if (groups != 0xFu && g->path_mask == nullptr) return EQUITP_INVALID_ARG;
  if (x == nullptr || W1 == nullptr || W2 == nullptr || grad_out == nullptr) return EQUITP_INVALID_ARG;
  if (g->n_edges > 0 && vec == nullptr) return EQUITP_INVALID_ARG;
  if (!aligned16(x) || !aligned16(grad_out) || (grad_x && !aligned16(grad_x)))
    return EQUITP_INVALID_ARG;
  if (grad_x && g->n_edges > 0 && (g->t_row_ptr == nullptr || g->t_perm == nullptr))
    return EQUITP_INVALID_ARG;
  if (grad_x && g->n_nodes > 0 && g->t_row_ptr == nullptr) return EQUITP_INVALID_ARG;
  if (int ms = mask_status(h->shape, g)) return ms;
  const int n_cu = n_cu_of_current_device();
  if (n_cu <= 0) return EQUITP_HIP_ERROR;
  const equitp::ConvShape& s = h->shape;
  const BwdLayout L = bwd_layout(s, g->n_edges, n_cu);
  const bool need_edge = (grad_vec != nullptr || grad_W1 != nullptr) && g->n_edges > 0;
  const bool need_dw2 = grad_W2 != nullptr && g->n_edges > 0;
  if ((need_edge || need_dw2) && (workspace == nullptr || workspace_bytes < L.total))
    return EQUITP_WORKSPACE_TOO_SMALL;
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return EQUITP_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  hipError_t err = hipSuccess;

  if (need_edge || need_dw2) {
    equitp::BwdParams b{};
    b.n_edges = g->n_edges;
    b.C = s.C;
    b.n_slices = s.C / 16;
    b.wg_per_slice = L.wps;
    b.src = g->src;
    b.dst = g->dst;
    b.vec = vec;
    b.x = x;
    b.G = grad_out;
    b.W1 = W1;
    b.W2 = W2;
    b.dvec_part = grad_vec ? reinterpret_cast<float*>(ws + L.dvec) : nullptr;
    b.dW2_part = grad_W2 ? reinterpret_cast<float*>(ws + L.dw2) : nullptr;
    b.dW1_part = grad_W1 ? reinterpret_cast<float*>(ws + L.dw1) : nullptr;
    b.inv_r_cut = 1.0f / s.r_cut;
    b.radial_pref = std::sqrt(2.0f / s.r_cut);
    b.path_mask = g->path_mask;
    if (g->path_mask != nullptr) {
      ProfScope ps("tile_order", st);
      b.n_tiles = (g->n_edges + 15) / 16;
      int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
      b.tile_order = tiles;
      err = uniform_mask ? (tiles_ready ? hipSuccess : equitp::launch_iota(tiles, b.n_tiles, st))
                         : equitp::launch_tile_order(g->n_edges, g->path_mask, tiles, ws + L.sort,
                                                     L.sort_bytes, st);
      if (err != hipSuccess) return EQUITP_HIP_ERROR;
    }
    if (groups != 0xFu) {
      // what the skipped groups would have started or written
      if (!(groups & 1u) && b.dvec_part)
        err = equitp::launch_fill_zero(b.dvec_part, (size_t)b.n_slices * g->n_edges * 3, st);
      if (err == hipSuccess && !(groups & 1u) && b.dW1_part)
        err = equitp::launch_fill_zero(b.dW1_part, (size_t)L.grid * s.n_radial * s.hidden, st);
      if (err == hipSuccess && b.dW2_part)
        err = equitp::launch_fill_zero(b.dW2_part, (size_t)L.wps * s.hidden * s.n_paths * s.C, st);
      if (err != hipSuccess) return EQUITP_HIP_ERROR;
    }
    {
      ProfScope ps("bwd", st);
      err = !b.path_mask         ? equitp::launch_bwd(s, b, st)
            : groups == 0xFu     ? equitp::launch_bwd_masked(s, b, st)
                                 : equitp::launch_bwd_masked_groups(s, b, groups, st);
    }
    if (err != hipSuccess) return EQUITP_HIP_ERROR;
    if (grad_vec) {
      ProfScope ps("sum_dvec", st);
      err = equitp::launch_sum_slices(b.dvec_part, b.n_slices, g->n_edges * 3, grad_vec, st);
      if (err != hipSuccess) return EQUITP_HIP_ERROR;
    }
    if (grad_W1) {
      ProfScope ps("reduce_dW1", st);
      err = equitp::launch_reduce_rows(b.dW1_part, L.grid, s.n_radial * s.hidden,
                                       grad_W1, st);
      if (err != hipSuccess) return EQUITP_HIP_ERROR;
    }
    if (grad_W2) {
      ProfScope ps("reduce_dW2", st);
      err = equitp::launch_reduce_rows(b.dW2_part, L.wps, s.hidden * s.n_paths * s.C, grad_W2, st);
      if (err != hipSuccess) return EQUITP_HIP_ERROR;
    }
  }
  if (!need_edge && grad_W1) {
    if ((err = equitp::launch_fill_zero(grad_W1, (size_t)s.n_radial * s.hidden, st)) != hipSuccess)
      return EQUITP_HIP_ERROR;
  }
  if (!need_dw2 && grad_W2) {
    if ((err = equitp::launch_fill_zero(grad_W2, (size_t)s.hidden * s.n_paths * s.C, st)) != hipSuccess)
      return EQUITP_HIP_ERROR;
  }

  if (grad_x != nullptr && g->n_nodes > 0) {
    equitp::SegParams p{};
    p.n_seg = g->n_nodes;
    p.C = s.C;
    p.n_slices = s.C / 16;
    p.seg_ptr = g->t_row_ptr;
    p.seg_edge = g->t_perm;
    p.gather = g->dst;
    p.vec = vec;
    p.feat = grad_out;
    p.W1 = W1;
    p.W2 = W2;
    p.out = grad_x;
    p.inv_r_cut = 1.0f / s.r_cut;
    p.radial_pref = std::sqrt(2.0f / s.r_cut);
    p.path_mask = g->path_mask;
    {
      ProfScope ps("seg_dx", st);
      err = p.path_mask ? equitp::launch_seg_conv_masked(s, true, p, n_cu, st)
                        : equitp::launch_seg_conv(s, true, p, n_cu, st);
    }
    if (err != hipSuccess) return EQUITP_HIP_ERROR;
  }
  return EQUITP_OK;
}

}  // namespace

int equitp_backward(equitp_t h, const equitp_graph* g, const float* vec, const float* x,
                    const float* W1, const float* W2, const float* grad_out, float* grad_vec,
                    float* grad_x, float* grad_W1, float* grad_W2, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return backward_impl(h, g, vec, x, W1, W2, grad_out, grad_vec, grad_x, grad_W1, grad_W2,
                       workspace, workspace_bytes, stream, 0xFu, false);
}

int equitp_linear(int n_nodes, int lmax, int channels, const float* feat_in, const float* W,
                  int transpose_w, float* out, void* stream) {
  if (n_nodes < 0 || lmax < 0 || lmax > 3) return EQUITP_INVALID_ARG;
  if (n_nodes == 0) return EQUITP_OK;
  if (feat_in == nullptr || W == nullptr || out == nullptr || feat_in == out) return EQUITP_INVALID_ARG;
  if (channels != 16 && channels != 32 && channels != 64 && channels != 128) return EQUITP_UNSUPPORTED;
  ProfScope ps("linear", (hipStream_t)stream);
  return hip_status(equitp::launch_linear(n_nodes, lmax, channels, feat_in, W, transpose_w, out,
                                          (hipStream_t)stream));
}

int equitp_build_csr_workspace(int n_nodes, int n_edges, size_t* bytes) {
  if (bytes == nullptr || n_nodes < 0 || n_edges < 0) return EQUITP_INVALID_ARG;
  *bytes = equitp::csr_workspace_bytes(n_nodes, n_edges);
  return EQUITP_OK;
}

int equitp_build_csr(int n_nodes, int n_edges, const int32_t* key, int32_t* row_ptr,
                     int32_t* perm, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_nodes < 0 || n_edges < 0 || row_ptr == nullptr) return EQUITP_INVALID_ARG;
  if (n_edges > 0 && (key == nullptr || perm == nullptr)) return EQUITP_INVALID_ARG;
  if (workspace_bytes < equitp::csr_workspace_bytes(n_nodes, n_edges) || workspace == nullptr)
    return EQUITP_WORKSPACE_TOO_SMALL;
  return hip_status(equitp::launch_build_csr(n_nodes, n_edges, key, row_ptr, perm, workspace,
                                             workspace_bytes, (hipStream_t)stream));
}

int equitp_cg_block(int l1, int l2, int l3, float* dense) {
  if (dense == nullptr) return EQUITP_INVALID_ARG;
  for (int p = 0; p < equitp::cg::kNumPaths; ++p) {
    const auto& P = equitp::cg::kPaths[p];
    if (P.l1 == l1 && P.l2 == l2 && P.l3 == l3) {
      const int d2 = 2 * l2 + 1, d3 = 2 * l3 + 1;
      std::memset(dense, 0, sizeof(float) * (2 * l1 + 1) * d2 * d3);
      for (int k = 0; k < P.nnz; ++k) {
        const auto& e = equitp::cg::kEnt[P.off + k];
        dense[(e.m1 * d2 + e.m2) * d3 + e.m3] = equitp::cg::kVal[P.off + k];
      }
      return EQUITP_OK;
    }
  }
  return EQUITP_UNSUPPORTED;
}

void equitp_destroy(equitp_t h) { delete h; }

int equitp_ladder_num_paths(int lmax, int* n_paths) {
  if (n_paths == nullptr) return EQUITP_INVALID_ARG;
  if (lmax < 0 || lmax > 3) return EQUITP_UNSUPPORTED;
  *n_paths = equitp::ladder_num_paths(lmax);
  return EQUITP_OK;
}

int equitp_ladder_forward(int lmax, int nu, int n_nodes, int channels, const float* A,
                          const float* w, float* out, float* rungs, void* stream) {
  equitp::LadderParams p;
  int st = ladder_layout(lmax, nu, n_nodes, channels, 256, &p);
  if (st != EQUITP_OK) return st;
  if (n_nodes == 0) return EQUITP_OK;
  if (A == nullptr || w == nullptr || out == nullptr || out == A) return EQUITP_INVALID_ARG;
  if (rungs != nullptr && (rungs == out || rungs == A)) return EQUITP_INVALID_ARG;
  p.A = A;
  p.w = w;
  p.out = out;
  p.rungs = nu > 2 ? rungs : nullptr;
  ProfScope ps("ladder_fwd", (hipStream_t)stream);
  return hip_status(equitp::launch_ladder_fwd(lmax, nu, p, (hipStream_t)stream));
}

int equitp_ladder_backward_workspace(int lmax, int nu, int n_nodes, int channels, size_t* bytes) {
  if (bytes == nullptr) return EQUITP_INVALID_ARG;
  equitp::LadderParams p;
  int st = ladder_layout(lmax, nu, n_nodes, channels, n_cu_of_current_device(), &p);
  if (st != EQUITP_OK) return st;
  *bytes = ladder_workspace_bytes(p, lmax, nu);
  return EQUITP_OK;
}

int equitp_ladder_backward(int lmax, int nu, int n_nodes, int channels, const float* A,
                           const float* w, const float* rungs, const float* grad_out, float* grad_A,
                           float* grad_w, void* workspace, size_t workspace_bytes, void* stream) {
  equitp::LadderParams p;
  int st = ladder_layout(lmax, nu, n_nodes, channels, n_cu_of_current_device(), &p);
  if (st != EQUITP_OK) return st;
  const hipStream_t hs = (hipStream_t)stream;
  const size_t n_w = (size_t)(nu - 1) * equitp::ladder_num_paths(lmax) * channels;
  if (n_nodes == 0) {
    if (grad_w == nullptr) return EQUITP_OK;
    return hip_status(equitp::launch_fill_zero(grad_w, n_w, hs));
  }
  if (A == nullptr || w == nullptr || grad_out == nullptr) return EQUITP_INVALID_ARG;
  if (grad_A != nullptr && (grad_A == A || grad_A == grad_out || (rungs && grad_A == rungs)))
    return EQUITP_INVALID_ARG;
  if (grad_w != nullptr) {
    if (workspace == nullptr || workspace_bytes < ladder_workspace_bytes(p, lmax, nu))
      return EQUITP_WORKSPACE_TOO_SMALL;
  }
  p.A = A;
  p.w = w;
  p.G = grad_out;
  p.dA = grad_A;
  p.dw_part = static_cast<float*>(workspace);
  p.rungs = nu > 2 ? const_cast<float*>(rungs) : nullptr;   // read only in the backward
  {
    ProfScope ps("ladder_bwd", hs);
    hipError_t e = equitp::launch_ladder_bwd(lmax, nu, p, grad_A != nullptr, grad_w != nullptr, hs);
    if (e != hipSuccess) return EQUITP_HIP_ERROR;
  }
  if (grad_w != nullptr) {
    ProfScope ps("ladder_reduce_dw", hs);
    float* tmp = reinterpret_cast<float*>(static_cast<char*>(workspace) + ladder_part_bytes(p, lmax, nu));
    return hip_status(equitp::launch_ladder_reduce(p.dw_part, p.blocks_per_group, (int)n_w, tmp,
                                                   grad_w, hs));
  }
  return EQUITP_OK;
}

// ---------------------------------------------------------------- full product ladder
namespace {

struct FullLayout {
  size_t nfc, t_floats, lev_floats, gs_floats, part_floats;
  size_t bytes() const { return (t_floats + lev_floats + gs_floats + part_floats) * sizeof(float); }
};

int full_layout(int lmax, int nu, int n_nodes, int channels, bool backward, FullLayout* f) {
  if (n_nodes < 0 || channels <= 0) return EQUITP_INVALID_ARG;
  if (lmax < 0 || lmax > 3 || nu < 2 || nu > 5 || !equitp::full_ladder_channels_ok(channels) ||
      n_nodes > (1 << 26))
    return EQUITP_UNSUPPORTED;
  const size_t N = (size_t)n_nodes, C = (size_t)channels, F = (size_t)(lmax + 1) * (lmax + 1);
  f->nfc = N * F * C;
  // every size rounded to 64 floats (256 bytes) so each carved buffer stays aligned
  auto up = [](size_t n) { return (n + 63) & ~size_t(63); };
  f->t_floats = up(N * (size_t)equitp::full_ladder_dsum(lmax) * C);
  if (!backward) {
    f->lev_floats = up((size_t)std::min(2, nu - 2) * f->nfc);
    f->gs_floats = f->part_floats = 0;
  } else {
    f->lev_floats = up((size_t)(nu - 2) * f->nfc);
    f->gs_floats = nu > 2 ? up(f->nfc) : 0;
    f->part_floats = up((size_t)equitp::full_ladder_dw_blocks(lmax, n_nodes, channels) * C * C);
  }
  return EQUITP_OK;
}

}  // namespace

int equitp_full_ladder_workspace(int lmax, int nu, int n_nodes, int channels, int backward,
                                 size_t* bytes) {
  if (bytes == nullptr) return EQUITP_INVALID_ARG;
  FullLayout f;
  int st = full_layout(lmax, nu, n_nodes, channels, backward != 0, &f);
  if (st != EQUITP_OK) return st;
  *bytes = f.bytes();
  return EQUITP_OK;
}

int equitp_full_ladder_saved_floats(int lmax, int nu, int n_nodes, int channels, size_t* n) {
  if (n == nullptr) return EQUITP_INVALID_ARG;
  FullLayout f;
  int st = full_layout(lmax, nu, n_nodes, channels, false, &f);
  if (st != EQUITP_OK) return st;
  *n = (size_t)(nu - 1) * n_nodes * equitp::full_ladder_dsum(lmax) * channels;
  return EQUITP_OK;
}

int equitp_full_ladder_forward(int lmax, int nu, int n_nodes, int channels, const float* A,
                               const float* W, float* out, float* rungs, float* saved,
                               void* workspace, size_t workspace_bytes, void* stream) {
  FullLayout f;
  int st = full_layout(lmax, nu, n_nodes, channels, false, &f);
  if (st != EQUITP_OK) return st;
  if (n_nodes == 0) return EQUITP_OK;
  if (A == nullptr || W == nullptr || out == nullptr || out == A) return EQUITP_INVALID_ARG;
  if (rungs != nullptr && (rungs == out || rungs == A)) return EQUITP_INVALID_ARG;
  if (saved != nullptr && (saved == out || saved == A || saved == rungs)) return EQUITP_INVALID_ARG;
  // the GEMM stages 16-byte vectors of every operand
  if (!aligned16(A) || !aligned16(W) || !aligned16(out) || (rungs && !aligned16(rungs)) ||
      (saved && !aligned16(saved)) || (workspace && !aligned16(workspace)))
    return EQUITP_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < f.bytes()) return EQUITP_WORKSPACE_TOO_SMALL;
  const hipStream_t hs = (hipStream_t)stream;
  float* T = static_cast<float*>(workspace);
  float* lev = T + f.t_floats;
  const size_t wstep = (size_t)equitp::ladder_num_paths(lmax) * channels * channels;
  auto level = [&](int s) -> float* {   // B_s, s = 2 .. nu-1
    return rungs ? rungs + (size_t)(s - 2) * f.nfc : lev + (size_t)((s - 2) % 2) * f.nfc;
  };
  const size_t tstep = (size_t)n_nodes * equitp::full_ladder_dsum(lmax) * channels;
  for (int s = 2; s <= nu; ++s) {
    const float* Bp = s == 2 ? A : level(s - 1);
    float* Ts = saved ? saved + (size_t)(s - 2) * tstep : T;   // this step's path outputs
    {
      ProfScope ps("full_tp", hs);
      if (equitp::launch_full_tp(lmax, n_nodes, channels, Bp, A, Ts, hs) != hipSuccess)
        return EQUITP_HIP_ERROR;
    }
    ProfScope ps("mix_fwd", hs);
    if (equitp::launch_mix_fwd(lmax, n_nodes, channels, Ts, W + (size_t)(s - 2) * wstep, out, s > 2,
                               s < nu ? level(s) : nullptr, hs) != hipSuccess)
      return EQUITP_HIP_ERROR;
  }
  return EQUITP_OK;
}

int equitp_full_ladder_backward(int lmax, int nu, int n_nodes, int channels, const float* A,
                                const float* W, const float* rungs, const float* saved,
                                const float* grad_out, float* grad_A, float* grad_W,
                                void* workspace, size_t workspace_bytes, void* stream) {
  FullLayout f;
  int st = full_layout(lmax, nu, n_nodes, channels, true, &f);
  if (st != EQUITP_OK) return st;
  const hipStream_t hs = (hipStream_t)stream;
  const size_t wstep = (size_t)equitp::ladder_num_paths(lmax) * channels * channels;
  if (n_nodes == 0) {
    if (grad_W == nullptr) return EQUITP_OK;
    return hip_status(equitp::launch_fill_zero(grad_W, (size_t)(nu - 1) * wstep, hs));
  }
  if (A == nullptr || W == nullptr || grad_out == nullptr) return EQUITP_INVALID_ARG;
  if (grad_A != nullptr && (grad_A == A || grad_A == grad_out || (rungs && grad_A == rungs)))
    return EQUITP_INVALID_ARG;
  if (grad_A == nullptr && grad_W == nullptr) return EQUITP_OK;
  if (!aligned16(A) || !aligned16(W) || !aligned16(grad_out) || (rungs && !aligned16(rungs)) ||
      (saved && !aligned16(saved)) || (grad_A && !aligned16(grad_A)) ||
      (grad_W && !aligned16(grad_W)) || (workspace && !aligned16(workspace)))
    return EQUITP_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < f.bytes()) return EQUITP_WORKSPACE_TOO_SMALL;
  float* T = static_cast<float*>(workspace);
  float* lev = T + f.t_floats;
  float* Gsb = lev + f.lev_floats;
  float* part = Gsb + f.gs_floats;
  const float* lv = rungs ? rungs : lev;
  auto level = [&](int s) -> const float* { return lv + (size_t)(s - 2) * f.nfc; };
  if (rungs == nullptr) {
    // B_2 .. B_{nu-1} again, kept whole this time
    for (int s = 2; s < nu; ++s) {
      const float* Bp = s == 2 ? A : level(s - 1);
      {
        ProfScope ps("full_tp", hs);
        if (equitp::launch_full_tp(lmax, n_nodes, channels, Bp, A, T, hs) != hipSuccess)
          return EQUITP_HIP_ERROR;
      }
      ProfScope ps("mix_fwd", hs);
      if (equitp::launch_mix_fwd(lmax, n_nodes, channels, T, W + (size_t)(s - 2) * wstep, nullptr,
                                 false, lev + (size_t)(s - 2) * f.nfc, hs) != hipSuccess)
        return EQUITP_HIP_ERROR;
    }
  }
  const float* Gs = grad_out;
  bool first = true;
  for (int s = nu; s >= 2; --s) {
    const float* Bp = s == 2 ? A : level(s - 1);
    const float* Ws = W + (size_t)(s - 2) * wstep;
    if (grad_W != nullptr) {
      // this step's path outputs: kept by the forward, or computed again
      const float* Ts = saved ? saved + (size_t)(s - 2) * n_nodes * equitp::full_ladder_dsum(lmax) * channels
                              : T;
      if (saved == nullptr) {
        ProfScope ps("full_tp", hs);
        if (equitp::launch_full_tp(lmax, n_nodes, channels, Bp, A, T, hs) != hipSuccess)
          return EQUITP_HIP_ERROR;
      }
      ProfScope ps("mix_dw", hs);
      if (equitp::launch_mix_dw(lmax, n_nodes, channels, Ts, Gs, part,
                                grad_W + (size_t)(s - 2) * wstep, hs) != hipSuccess)
        return EQUITP_HIP_ERROR;
    }
    if (s == 2 && grad_A == nullptr) break;
    {
      ProfScope ps("mix_dt", hs);
      if (equitp::launch_mix_dt(lmax, n_nodes, channels, Gs, Ws, T, hs) != hipSuccess)
        return EQUITP_HIP_ERROR;
    }
    ProfScope ps("full_tp_bwd", hs);
    if (equitp::launch_full_tp_bwd(lmax, n_nodes, channels, Bp, A, T, grad_out,
                                   s > 2 ? Gsb : nullptr, grad_A, !first, s == 2, hs) != hipSuccess)
      return EQUITP_HIP_ERROR;
    if (grad_A != nullptr) first = false;
    Gs = Gsb;
  }
  return EQUITP_OK;
}

// ---------------------------------------------------------------- mixed multiplicities
// The convolution with its own channel count per rotation order is composed from the uniform
// kernels.  Channel slices: the distinct input multiplicities t_1 < t_2 < ... cut the channels into
// slices [t_{k-1}, t_k), uniform in width, in which exactly the ranks with m_in[l] >= t_k have
// channels.  Per slice, the masked convolution keeps one path per output rank in each launch, so
// its output block l3 is that path's receiver sum; the blocks are copied into per-path rows
// zero-padded to Cp channels, and the full ladder's mixing GEMM (forward, dT and dW modes) applies
// the per-path maps, zero-padded to Cp x Cp.
struct equitp_mixed {
  int L = 0, H = 64, n_radial = 8;
  int mult_in[4] = {}, mult_out[4] = {};
  int off_in[4] = {}, off_out[4] = {}, row_in = 0, row_out = 0;
  int P = 0;
  int pl1[32] = {}, pl3[32] = {}, wcol[32] = {}, wlin_off[32] = {}, toff[32] = {};
  int w2cols = 0, wlin_numel = 0, dsum = 0, Cp = 128;
  int n_slices = 0;
  int t0[4] = {}, w[4] = {};
  equitp_t conv[4] = {};
  int n_launch[4] = {};
  int sel[4][8][4] = {};   // [slice][launch][l3]: path computed for that rank, or -1
  uint32_t mask[4][8] = {};
  // backward launches: one path group of the masked backward each (so the other groups' kernels
  // do not run), at most one path per output rank
  int bn_launch[4] = {};
  int bgroup[4][16] = {};
  int bsel[4][16][4] = {};
  uint32_t bmask[4][16] = {};
  ~equitp_mixed() {
    for (int k = 0; k < 4; ++k)
      if (conv[k]) equitp_destroy(conv[k]);
  }
};

namespace {

// "128x0e+64x1o+32x2e+32x3o": one block per l from 0 up, parity (-1)^l.
int parse_mixed(const char* s, int* L, int mult[4]) {
  std::vector<Block> b;
  if (!parse_irreps(s, b)) return EQUITP_IRREPS_PARSE;
  if (b.size() > 4) return EQUITP_UNSUPPORTED;
  for (size_t i = 0; i < b.size(); ++i) {
    if (b[i].l != (int)i || b[i].parity != ((i % 2) ? -1 : 1)) return EQUITP_UNSUPPORTED;
    if (b[i].mul <= 0 || b[i].mul % 32 != 0 || b[i].mul > 128) return EQUITP_UNSUPPORTED;
    mult[i] = b[i].mul;
  }
  *L = (int)b.size() - 1;
  return EQUITP_OK;
}

struct MixedLayout {
  // forward
  size_t xs[4], w2s[4], mask, outl, T, Wpad, opad;
  // backward
  size_t gpad, part, dwpad, gl, dvec_j, dx_j, dw1_j, dw2_j, dxs[4], dw2s[4], convws, convws_bytes;
  size_t total;
};

int mixed_layout(const equitp_mixed* h, int N, int E, bool backward, MixedLayout* m) {
  *m = MixedLayout{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) & ~size_t(255);
    return at;
  };
  const size_t F = (size_t)(h->L + 1) * (h->L + 1), Cp = h->Cp, f = sizeof(float);
  for (int k = 0; k < h->n_slices; ++k) {
    m->xs[k] = take((size_t)N * F * h->w[k] * f);
    m->w2s[k] = take((size_t)h->H * h->P * h->w[k] * f);
  }
  int wmax = 0;
  for (int k = 0; k < h->n_slices; ++k) wmax = std::max(wmax, h->w[k]);
  m->mask = take((size_t)E * sizeof(uint32_t));
  m->outl = take((size_t)N * F * wmax * f);
  m->T = take((size_t)N * h->dsum * Cp * f);
  m->Wpad = take((size_t)h->P * Cp * Cp * f);
  m->opad = take((size_t)N * F * Cp * f);
  if (backward) {
    m->gpad = take((size_t)N * F * Cp * f);
    m->part = take((size_t)equitp::full_ladder_dw_blocks(h->L, N, (int)Cp) * Cp * Cp * f);
    m->dwpad = take((size_t)h->P * Cp * Cp * f);
    m->gl = take((size_t)N * F * wmax * f);
    m->dvec_j = take((size_t)E * 3 * f);
    m->dx_j = take((size_t)N * F * wmax * f);
    m->dw1_j = take((size_t)h->n_radial * h->H * f);
    m->dw2_j = take((size_t)h->H * h->P * wmax * f);
    for (int k = 0; k < h->n_slices; ++k) {
      m->dxs[k] = take((size_t)N * F * h->w[k] * f);
      m->dw2s[k] = take((size_t)h->H * h->P * h->w[k] * f);
    }
    size_t cw = 0;
    for (int k = 0; k < h->n_slices; ++k) {
      size_t b = 0;
      int st = equitp_backward_workspace(h->conv[k], N, E, &b);
      if (st != EQUITP_OK) return st;
      cw = std::max(cw, b);
    }
    m->convws_bytes = cw;
    m->convws = take(cw);
  }
  m->total = o;
  return EQUITP_OK;
}

equitp::RowMap plain(float* base, long long ld, long long off = 0) {
  return equitp::RowMap{base, 1, ld, off, 0};
}
// rows (n, m) of rank l in the uniform layout [N][F][C]
equitp::RowMap uniform_rows(float* base, int F, int C, int l) {
  return equitp::RowMap{base, 2 * l + 1, (long long)F * C, (long long)l * l * C, C};
}
// rows (n, m) of rank l in a mixed node tensor
equitp::RowMap mixed_rows(float* base, int row_len, int off_l, int mult_l, int l) {
  return equitp::RowMap{base, 2 * l + 1, row_len, off_l, mult_l};
}

#define MX_CHECK(expr)                                   \
  do {                                                   \
    if ((expr) != hipSuccess) return EQUITP_HIP_ERROR;   \
  } while (0)

using equitp::CopyJob;

// The input slices [N][(L+1)^2][w] (ranks a slice does not carry stay zero) and the slices' W2
// [H][P w] (columns of paths a slice does not carry stay zero).
int mixed_slices_in(const equitp_mixed* h, int N, const float* x, const float* W2, char* ws,
                    const MixedLayout& m, hipStream_t st) {
  const int F = (h->L + 1) * (h->L + 1);
  ProfScope ps("mixed_repack", st);
  std::vector<CopyJob> jobs;
  for (int k = 0; k < h->n_slices; ++k) {
    const int wk = h->w[k], hi = h->t0[k] + wk;
    float* xs = reinterpret_cast<float*>(ws + m.xs[k]);
    float* w2s = reinterpret_cast<float*>(ws + m.w2s[k]);
    MX_CHECK(equitp::launch_fill_zero(xs, (size_t)N * F * wk, st));
    MX_CHECK(equitp::launch_fill_zero(w2s, (size_t)h->H * h->P * wk, st));
    for (int l = 0; l <= h->L; ++l)
      if (h->mult_in[l] >= hi)
        jobs.push_back({uniform_rows(xs, F, wk, l),
                        mixed_rows(const_cast<float*>(x), h->row_in, h->off_in[l] + h->t0[k],
                                   h->mult_in[l], l),
                        N * (2 * l + 1), wk});
    for (int p = 0; p < h->P; ++p)
      if (h->mult_in[h->pl1[p]] >= hi)
        jobs.push_back({plain(w2s, (long long)h->P * wk, (long long)p * wk),
                        plain(const_cast<float*>(W2), h->w2cols, h->wcol[p] + h->t0[k]), h->H, wk});
  }
  MX_CHECK(equitp::launch_copy_batch(jobs.data(), (int)jobs.size(), st));
  return EQUITP_OK;
}

// Rows of path p's outputs (or their gradients) for channel slice k inside the padded per-path
// rows [N (2 l3 + 1)][Cp] of path p.
equitp::RowMap path_rows(const equitp_mixed* h, float* T, int N, int p, int k) {
  const int d = 2 * h->pl3[p] + 1;
  return equitp::RowMap{T, d, (long long)d * h->Cp, (long long)h->toff[p] * N * h->Cp + h->t0[k],
                        h->Cp};
}

// Path outputs of every path, per-path rows zero-padded to Cp channels, into T (the input slices
// must be in the workspace).
int mixed_path_outputs(const equitp_mixed* h, const equitp_graph* g, const float* vec,
                       const float* W1, float* T, char* ws, const MixedLayout& m, hipStream_t st) {
  const int N = g->n_nodes, E = g->n_edges, F = (h->L + 1) * (h->L + 1), Cp = h->Cp;
  uint32_t* mask = reinterpret_cast<uint32_t*>(ws + m.mask);
  float* outl = reinterpret_cast<float*>(ws + m.outl);
  MX_CHECK(equitp::launch_fill_zero(T, (size_t)N * h->dsum * Cp, st));
  for (int k = 0; k < h->n_slices; ++k) {
    const int wk = h->w[k];
    for (int j = 0; j < h->n_launch[k]; ++j) {
      MX_CHECK(equitp::launch_fill_u32(mask, (size_t)E, h->mask[k][j], st));
      equitp_graph gm = *g;
      gm.path_mask = mask;
      int s2 = equitp_forward(h->conv[k], &gm, vec, reinterpret_cast<float*>(ws + m.xs[k]), W1,
                              reinterpret_cast<float*>(ws + m.w2s[k]), outl, st);
      if (s2 != EQUITP_OK) return s2;
      ProfScope ps("mixed_repack", st);
      CopyJob jobs[4];
      int n = 0;
      for (int l3 = 0; l3 <= h->L; ++l3) {
        const int p = h->sel[k][j][l3];
        if (p >= 0) jobs[n++] = {path_rows(h, T, N, p, k), uniform_rows(outl, F, wk, l3), N * (2 * l3 + 1), wk};
      }
      MX_CHECK(equitp::launch_copy_batch(jobs, n, st));
    }
  }
  return EQUITP_OK;
}

// Per-path maps zero-padded to Cp x Cp.
int mixed_pad_maps(const equitp_mixed* h, const float* Wlin, float* Wpad, hipStream_t st) {
  const int Cp = h->Cp;
  ProfScope ps("mixed_repack", st);
  MX_CHECK(equitp::launch_fill_zero(Wpad, (size_t)h->P * Cp * Cp, st));
  std::vector<CopyJob> jobs;
  for (int p = 0; p < h->P; ++p)
    jobs.push_back({plain(Wpad, Cp, (long long)p * Cp * Cp),
                    plain(const_cast<float*>(Wlin), h->mult_out[h->pl3[p]], h->wlin_off[p]),
                    h->mult_in[h->pl1[p]], h->mult_out[h->pl3[p]]});
  MX_CHECK(equitp::launch_copy_batch(jobs.data(), (int)jobs.size(), st));
  return EQUITP_OK;
}

}  // namespace

int equitp_mixed_create(const char* irreps_in, const char* irreps_out, int n_radial, int hidden,
                        float r_cut, equitp_mixed_t* out) {
  if (out == nullptr) return EQUITP_INVALID_ARG;
  *out = nullptr;
  int Li, Lo, mi[4] = {}, mo[4] = {};
  int st;
  if ((st = parse_mixed(irreps_in, &Li, mi)) != EQUITP_OK) return st;
  if ((st = parse_mixed(irreps_out, &Lo, mo)) != EQUITP_OK) return st;
  if (!(r_cut > 0.0f) || n_radial <= 0) return EQUITP_INVALID_ARG;
  if (Li != Lo || Li < 1 || n_radial != 8 || hidden != 64) return EQUITP_UNSUPPORTED;
  equitp_mixed* h = new (std::nothrow) equitp_mixed();
  if (h == nullptr) return EQUITP_INVALID_ARG;
  h->L = Li;
  h->H = hidden;
  h->n_radial = n_radial;
  int mmax = 0;
  for (int l = 0; l <= h->L; ++l) {
    h->mult_in[l] = mi[l];
    h->mult_out[l] = mo[l];
    h->off_in[l] = h->row_in;
    h->off_out[l] = h->row_out;
    h->row_in += (2 * l + 1) * mi[l];
    h->row_out += (2 * l + 1) * mo[l];
    mmax = std::max(mmax, std::max(mi[l], mo[l]));
  }
  h->Cp = mmax <= 32 ? 32 : (mmax <= 64 ? 64 : 128);
  // paths in the convolution's order (lexicographic, triangle rule, l1 + l2 + l3 even)
  for (int l1 = 0; l1 <= h->L; ++l1)
    for (int l2 = 0; l2 <= h->L; ++l2)
      for (int l3 = std::abs(l1 - l2); l3 <= std::min(l1 + l2, h->L); ++l3)
        if ((l1 + l2 + l3) % 2 == 0) {
          const int p = h->P++;
          h->pl1[p] = l1;
          h->pl3[p] = l3;
          h->wcol[p] = h->w2cols;
          h->w2cols += mi[l1];
          h->wlin_off[p] = h->wlin_numel;
          h->wlin_numel += mi[l1] * mo[l3];
          h->toff[p] = h->dsum;
          h->dsum += 2 * l3 + 1;
        }
  // channel slices between consecutive distinct input multiplicities
  int thr[4], nt = 0;
  for (int l = 0; l <= h->L; ++l) {
    bool seen = false;
    for (int i = 0; i < nt; ++i) seen = seen || thr[i] == mi[l];
    if (!seen) thr[nt++] = mi[l];
  }
  std::sort(thr, thr + nt);
  std::string sh;
  for (int l = 0; l <= h->L; ++l) sh += (l ? "+1x" : "1x") + std::to_string(l) + (l % 2 ? "o" : "e");
  for (int k = 0; k < nt; ++k) {
    h->t0[k] = k ? thr[k - 1] : 0;
    h->w[k] = thr[k] - h->t0[k];
    std::string ir;
    for (int l = 0; l <= h->L; ++l)
      ir += (l ? "+" : "") + std::to_string(h->w[k]) + "x" + std::to_string(l) + (l % 2 ? "o" : "e");
    if ((st = equitp_create(ir.c_str(), sh.c_str(), ir.c_str(), n_radial, &h->conv[k])) != EQUITP_OK ||
        (st = equitp_set_radial(h->conv[k], hidden, r_cut)) != EQUITP_OK) {
      delete h;
      return st;
    }
    ++h->n_slices;
    // launches: the j-th path of each output rank (among the paths this slice carries)
    int cnt[4] = {};
    for (int j = 0; j < 8; ++j)
      for (int l3 = 0; l3 < 4; ++l3) h->sel[k][j][l3] = -1;
    for (int p = 0; p < h->P; ++p) {
      if (mi[h->pl1[p]] < thr[k]) continue;
      const int j = cnt[h->pl3[p]]++;
      h->sel[k][j][h->pl3[p]] = p;
      h->mask[k][j] |= 1u << p;
      h->n_launch[k] = std::max(h->n_launch[k], j + 1);
    }
    for (int j = 0; j < 16; ++j)
      for (int l3 = 0; l3 < 4; ++l3) h->bsel[k][j][l3] = -1;
    for (int grp = 0; grp < 4; ++grp) {
      int c[4] = {}, most = 0;
      const int first = h->bn_launch[k];
      for (int p = 0; p < h->P; ++p) {
        if (mi[h->pl1[p]] < thr[k] || equitp::bwd_path_group(h->L, p) != grp) continue;
        const int j = first + c[h->pl3[p]]++;
        if (j >= 16) {
          delete h;
          return EQUITP_UNSUPPORTED;
        }
        h->bgroup[k][j] = grp;
        h->bsel[k][j][h->pl3[p]] = p;
        h->bmask[k][j] |= 1u << p;
        most = std::max(most, j + 1 - first);
      }
      h->bn_launch[k] = first + most;
    }
  }
  *out = h;
  return EQUITP_OK;
}

void equitp_mixed_destroy(equitp_mixed_t h) { delete h; }

int equitp_mixed_query(equitp_mixed_t h, int* n_paths, int* f_in, int* f_out, int* w2_numel,
                       int* wlin_numel, int* n_slices, int* n_launches) {
  if (h == nullptr) return EQUITP_INVALID_ARG;
  if (n_paths) *n_paths = h->P;
  if (f_in) *f_in = h->row_in;
  if (f_out) *f_out = h->row_out;
  if (w2_numel) *w2_numel = h->H * h->w2cols;
  if (wlin_numel) *wlin_numel = h->wlin_numel;
  if (n_slices) *n_slices = h->n_slices;
  if (n_launches) {   // forward launches per pass
    int n = 0;
    for (int k = 0; k < h->n_slices; ++k) n += h->n_launch[k];
    *n_launches = n;
  }
  return EQUITP_OK;
}

int equitp_mixed_workspace(equitp_mixed_t h, int n_nodes, int n_edges, int backward, size_t* bytes) {
  if (h == nullptr || bytes == nullptr || n_nodes < 0 || n_edges < 0) return EQUITP_INVALID_ARG;
  if (n_nodes > (1 << 24)) return EQUITP_UNSUPPORTED;
  MixedLayout m;
  int st = mixed_layout(h, n_nodes, n_edges, backward != 0, &m);
  if (st != EQUITP_OK) return st;
  *bytes = m.total;
  return EQUITP_OK;
}

int equitp_mixed_saved_floats(equitp_mixed_t h, int n_nodes, size_t* n) {
  if (h == nullptr || n == nullptr || n_nodes < 0) return EQUITP_INVALID_ARG;
  *n = (size_t)n_nodes * h->dsum * h->Cp;
  return EQUITP_OK;
}

int equitp_mixed_forward(equitp_mixed_t h, const equitp_graph* g, const float* vec, const float* x,
                         const float* W1, const float* W2, const float* Wlin, float* out,
                         float* saved, void* workspace, size_t workspace_bytes, void* stream) {
  if (h == nullptr || g == nullptr) return EQUITP_INVALID_ARG;
  if (g->n_nodes < 0 || g->n_edges < 0 || g->path_mask != nullptr) return EQUITP_INVALID_ARG;
  if (g->n_nodes > (1 << 24)) return EQUITP_UNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  const int N = g->n_nodes;
  if (N == 0) return EQUITP_OK;
  if (x == nullptr || W1 == nullptr || W2 == nullptr || Wlin == nullptr || out == nullptr ||
      (g->n_edges > 0 && vec == nullptr) || out == x || (saved && (saved == out || saved == x)))
    return EQUITP_INVALID_ARG;
  // repacks and GEMM use 16-byte vectors; the workspace is carved in 256-byte steps
  if (!aligned16(x) || !aligned16(W2) || !aligned16(Wlin) || !aligned16(out) ||
      (saved && !aligned16(saved)) || (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255)))
    return EQUITP_INVALID_ARG;
  MixedLayout m;
  int s2 = mixed_layout(h, N, g->n_edges, false, &m);
  if (s2 != EQUITP_OK) return s2;
  if (workspace == nullptr || workspace_bytes < m.total) return EQUITP_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  const int F = (h->L + 1) * (h->L + 1), Cp = h->Cp;
  float* T = saved ? saved : reinterpret_cast<float*>(ws + m.T);
  if ((s2 = mixed_slices_in(h, N, x, W2, ws, m, st)) != EQUITP_OK) return s2;
  if ((s2 = mixed_path_outputs(h, g, vec, W1, T, ws, m, st)) != EQUITP_OK) return s2;
  float* Wpad = reinterpret_cast<float*>(ws + m.Wpad);
  float* opad = reinterpret_cast<float*>(ws + m.opad);
  if ((s2 = mixed_pad_maps(h, Wlin, Wpad, st)) != EQUITP_OK) return s2;
  {
    ProfScope ps("mixed_mix_fwd", st);
    MX_CHECK(equitp::launch_mix_fwd(h->L, N, Cp, T, Wpad, opad, false, nullptr, st));
  }
  ProfScope ps("mixed_repack", st);
  CopyJob jobs[4];
  for (int l = 0; l <= h->L; ++l)
    jobs[l] = {mixed_rows(out, h->row_out, h->off_out[l], h->mult_out[l], l),
               uniform_rows(opad, F, Cp, l), N * (2 * l + 1), h->mult_out[l]};
  MX_CHECK(equitp::launch_copy_batch(jobs, h->L + 1, st));
  return EQUITP_OK;
}

int equitp_mixed_backward(equitp_mixed_t h, const equitp_graph* g, const float* vec,
                          const float* x, const float* W1, const float* W2, const float* Wlin,
                          const float* saved, const float* grad_out, float* grad_vec,
                          float* grad_x, float* grad_W1, float* grad_W2, float* grad_Wlin,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (h == nullptr || g == nullptr) return EQUITP_INVALID_ARG;
  if (g->n_nodes < 0 || g->n_edges < 0 || g->path_mask != nullptr) return EQUITP_INVALID_ARG;
  if (g->n_nodes > (1 << 24)) return EQUITP_UNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  const int N = g->n_nodes, E = g->n_edges;
  const bool conv_grads = grad_vec || grad_x || grad_W1 || grad_W2;
  if (!conv_grads && !grad_Wlin) return EQUITP_OK;
  if (N == 0) {
    if (grad_W1) MX_CHECK(equitp::launch_fill_zero(grad_W1, (size_t)h->n_radial * h->H, st));
    if (grad_W2) MX_CHECK(equitp::launch_fill_zero(grad_W2, (size_t)h->H * h->w2cols, st));
    if (grad_Wlin) MX_CHECK(equitp::launch_fill_zero(grad_Wlin, (size_t)h->wlin_numel, st));
    return EQUITP_OK;
  }
  if (x == nullptr || W1 == nullptr || W2 == nullptr || Wlin == nullptr || grad_out == nullptr ||
      (E > 0 && vec == nullptr))
    return EQUITP_INVALID_ARG;
  if (grad_x && (grad_x == x || grad_x == grad_out)) return EQUITP_INVALID_ARG;
  if (grad_x && (g->t_row_ptr == nullptr || (E > 0 && g->t_perm == nullptr)))
    return EQUITP_INVALID_ARG;
  if (!aligned16(x) || !aligned16(W2) || !aligned16(Wlin) || !aligned16(grad_out) ||
      (saved && !aligned16(saved)) || (grad_x && !aligned16(grad_x)) ||
      (grad_W2 && !aligned16(grad_W2)) || (grad_Wlin && !aligned16(grad_Wlin)) ||
      (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255)))
    return EQUITP_INVALID_ARG;
  MixedLayout m;
  int s2 = mixed_layout(h, N, E, true, &m);
  if (s2 != EQUITP_OK) return s2;
  if (workspace == nullptr || workspace_bytes < m.total) return EQUITP_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const int F = (h->L + 1) * (h->L + 1), Cp = h->Cp;
  float* Tws = fp(m.T);
  float* Gpad = fp(m.gpad);
  float* Wpad = fp(m.Wpad);
  if ((s2 = mixed_slices_in(h, N, x, W2, ws, m, st)) != EQUITP_OK) return s2;
  // the path outputs: kept by the forward, or computed again (dL/dWlin needs them)
  const float* T = saved;
  if (grad_Wlin && T == nullptr) {
    if ((s2 = mixed_path_outputs(h, g, vec, W1, Tws, ws, m, st)) != EQUITP_OK) return s2;
    T = Tws;
  }
  {
    ProfScope ps("mixed_repack", st);
    MX_CHECK(equitp::launch_fill_zero(Gpad, (size_t)N * F * Cp, st));
    CopyJob jobs[4];
    for (int l = 0; l <= h->L; ++l)
      jobs[l] = {uniform_rows(Gpad, F, Cp, l),
                 mixed_rows(const_cast<float*>(grad_out), h->row_out, h->off_out[l], h->mult_out[l], l),
                 N * (2 * l + 1), h->mult_out[l]};
    MX_CHECK(equitp::launch_copy_batch(jobs, h->L + 1, st));
  }
  if (grad_Wlin) {
    float* dWpad = fp(m.dwpad);
    {
      ProfScope ps("mixed_mix_dw", st);
      MX_CHECK(equitp::launch_mix_dw(h->L, N, Cp, T, Gpad, fp(m.part), dWpad, st));
    }
    ProfScope ps("mixed_repack", st);
    std::vector<CopyJob> jobs;
    for (int p = 0; p < h->P; ++p)
      jobs.push_back({plain(grad_Wlin, h->mult_out[h->pl3[p]], h->wlin_off[p]),
                      plain(dWpad, Cp, (long long)p * Cp * Cp), h->mult_in[h->pl1[p]],
                      h->mult_out[h->pl3[p]]});
    MX_CHECK(equitp::launch_copy_batch(jobs.data(), (int)jobs.size(), st));
  }
  if (!conv_grads) return EQUITP_OK;
  if ((s2 = mixed_pad_maps(h, Wlin, Wpad, st)) != EQUITP_OK) return s2;
  {
    ProfScope ps("mixed_mix_dt", st);
    MX_CHECK(equitp::launch_mix_dt(h->L, N, Cp, Gpad, Wpad, Tws, st));   // dL/dM, per path
  }
  if (grad_vec) MX_CHECK(equitp::launch_fill_zero(grad_vec, (size_t)E * 3, st));
  if (grad_W1) MX_CHECK(equitp::launch_fill_zero(grad_W1, (size_t)h->n_radial * h->H, st));
  float* gl = fp(m.gl);
  uint32_t* mask = reinterpret_cast<uint32_t*>(ws + m.mask);
  std::vector<CopyJob> scatter;
  for (int k = 0; k < h->n_slices; ++k) {
    // the identity tile order, written by the slice's first one-group call (the slices' handles
    // differ in width and paths, so each lays out the shared workspace differently)
    bool tiles_ready = false;
    const int wk = h->w[k], hi = h->t0[k] + wk;
    float* dxs = fp(m.dxs[k]);
    float* dw2s = fp(m.dw2s[k]);
    if (grad_x) MX_CHECK(equitp::launch_fill_zero(dxs, (size_t)N * F * wk, st));
    if (grad_W2) MX_CHECK(equitp::launch_fill_zero(dw2s, (size_t)h->H * h->P * wk, st));
    for (int j = 0; j < h->bn_launch[k]; ++j) {
      {
        ProfScope ps("mixed_repack", st);
        MX_CHECK(equitp::launch_fill_zero(gl, (size_t)N * F * wk, st));
        CopyJob jobs[4];
        int n = 0;
        for (int l3 = 0; l3 <= h->L; ++l3) {
          const int p = h->bsel[k][j][l3];
          if (p >= 0) jobs[n++] = {uniform_rows(gl, F, wk, l3), path_rows(h, Tws, N, p, k), N * (2 * l3 + 1), wk};
        }
        MX_CHECK(equitp::launch_copy_batch(jobs, n, st));
        MX_CHECK(equitp::launch_fill_u32(mask, (size_t)E, h->bmask[k][j], st));
      }
      equitp_graph gm = *g;
      gm.path_mask = mask;
      s2 = backward_impl(h->conv[k], &gm, vec, fp(m.xs[k]), W1, fp(m.w2s[k]), gl,
                         grad_vec ? fp(m.dvec_j) : nullptr, grad_x ? fp(m.dx_j) : nullptr,
                         grad_W1 ? fp(m.dw1_j) : nullptr, grad_W2 ? fp(m.dw2_j) : nullptr,
                         ws + m.convws, m.convws_bytes, st, 1u << h->bgroup[k][j], true,
                         tiles_ready);
      if (s2 != EQUITP_OK) return s2;
      tiles_ready = true;
      ProfScope ps("mixed_repack", st);
      if (grad_vec) MX_CHECK(equitp::launch_add(grad_vec, fp(m.dvec_j), (size_t)E * 3, st));
      if (grad_x) MX_CHECK(equitp::launch_add(dxs, fp(m.dx_j), (size_t)N * F * wk, st));
      if (grad_W1) MX_CHECK(equitp::launch_add(grad_W1, fp(m.dw1_j), (size_t)h->n_radial * h->H, st));
      if (grad_W2) MX_CHECK(equitp::launch_add(dw2s, fp(m.dw2_j), (size_t)h->H * h->P * wk, st));
    }
    if (grad_x)
      for (int l = 0; l <= h->L; ++l)
        if (h->mult_in[l] >= hi)
          scatter.push_back({mixed_rows(grad_x, h->row_in, h->off_in[l] + h->t0[k], h->mult_in[l], l),
                             uniform_rows(dxs, F, wk, l), N * (2 * l + 1), wk});
    if (grad_W2)
      for (int p = 0; p < h->P; ++p)
        if (h->mult_in[h->pl1[p]] >= hi)
          scatter.push_back({plain(grad_W2, h->w2cols, h->wcol[p] + h->t0[k]),
                             plain(dw2s, (long long)h->P * wk, (long long)p * wk), h->H, wk});
  }
  ProfScope ps("mixed_repack", st);
  MX_CHECK(equitp::launch_copy_batch(scatter.data(), (int)scatter.size(), st));
  return EQUITP_OK;
}

int equitp_profile_enable(int on) {
  g_prof_on = on != 0;
  return EQUITP_OK;
}

int equitp_profile_only(const char* names) {
  g_prof_only.clear();
  if (names != nullptr && names[0] != '\0') g_prof_only = "," + std::string(names) + ",";
  return EQUITP_OK;
}

int equitp_profile_reset(void) {
  for (auto& e : g_prof)
    for (auto& pr : e.ev) {
      g_ev_pool.push_back(pr.first);
      g_ev_pool.push_back(pr.second);
    }
  g_prof.clear();
  return EQUITP_OK;
}

int equitp_profile_count(void) { return (int)g_prof.size(); }

int equitp_profile_get(int i, const char** name, int* launches, double* total_ms) {
  if (i < 0 || i >= (int)g_prof.size()) return EQUITP_INVALID_ARG;
  ProfEntry& e = g_prof[i];
  for (auto& pr : e.ev) {
    if (hipEventSynchronize(pr.second) != hipSuccess) return EQUITP_HIP_ERROR;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return EQUITP_HIP_ERROR;
    e.total_ms += ms;
    e.launches += 1;
    g_ev_pool.push_back(pr.first);
    g_ev_pool.push_back(pr.second);
  }
  e.ev.clear();
  if (name) *name = e.name.c_str();
  if (launches) *launches = e.launches;
  if (total_ms) *total_ms = e.total_ms;
  return EQUITP_OK;
}

const char* equitp_status_string(int status) {
  switch (status) {
    case EQUITP_OK: return "ok";
    case EQUITP_INVALID_ARG: return "invalid argument";
    case EQUITP_IRREPS_PARSE: return "irreps string could not be parsed";
    case EQUITP_UNSUPPORTED: return "unsupported configuration";
    case EQUITP_HIP_ERROR: return "HIP runtime error";
    case EQUITP_WORKSPACE_TOO_SMALL: return "workspace too small";
    default: return "unknown status";
  }
}

}  // extern "C"

// C ABI of the convolution library (declarations and contracts in e3conv.h).
#include "e3conv.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "host_core.h"
#include "kernels.h"

using e3c::HostPath;
using e3c::Irrep;

struct e3conv_plan_s {
  int channels = 0;
  int lmax = 0;
  int num_x = 0, num_y = 0, num_out = 0;
  float avg = 1.0f;
  std::vector<Irrep> xin, out;
  std::vector<HostPath> paths;
  std::vector<std::vector<double>> cg;   // per path, [m1][m2][m3]
  // sparse export
  std::vector<int> ix, iy, ip, iout;
  std::vector<double> val;
  e3conv_ordering ordering = E3CONV_RECEIVER;
  // compiled kernels of the layout (nullptr if none) and of the plan's ordering
  const e3c::KernelSet* ks = nullptr;
  const e3c::OrderingKernels* kk = nullptr;
  int fwd_variant = 0;
  int bwd_variant = 0;
};

namespace {

thread_local std::string g_last_error;

e3conv_status fail(e3conv_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

e3conv_status ok() {
  g_last_error.clear();
  return E3CONV_OK;
}

e3conv_status hip_fail(hipError_t err, const char* what) {
  return fail(E3CONV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
}

}  // namespace

namespace e3c {
e3conv_status api_fail(e3conv_status st, const std::string& msg) { return fail(st, msg); }
e3conv_status api_ok() { return ok(); }
e3conv_status api_hip_fail(hipError_t err, const char* what) { return hip_fail(err, what); }
}  // namespace e3c

namespace {

// block code for kernel lookup: unique l in ascending order, else 0 (no kernel)
uint32_t block_code(const std::vector<Irrep>& blocks) {
  uint32_t code = 0;
  int prev = -1;
  for (const Irrep& b : blocks) {
    if (b.l <= prev || b.l > e3c::kMaxL) return 0;
    prev = b.l;
    code |= (b.parity > 0 ? 1u : 2u) << (2 * b.l);
  }
  return code;
}

// Pack the kernel coefficients in the kernel's enumeration order and check the
// host tables against it (paths identical, no nonzero outside the pattern).
bool bind_kernels(e3conv_plan_s* p, std::string* why) {
  const uint32_t xc = block_code(p->xin), oc = block_code(p->out);
  if (xc == 0 || oc == 0) return false;
  const e3c::KernelSet* ks = e3c::find_kernels(p->channels, xc, p->lmax, oc);
  if (!ks) return false;
  const e3c::LayoutTables& T = *ks->tables;
  if (T.num_paths != (int)p->paths.size() || T.num_x != p->num_x || T.num_out != p->num_out ||
      T.num_y != p->num_y) {
    *why = "kernel layout tables disagree with the host path enumeration";
    return false;
  }
  std::vector<double> coef(T.nnz, 0.0);
  for (int q = 0; q < T.num_paths; ++q) {
    const e3c::PathInfo& P = T.path[q];
    const HostPath& H = p->paths[q];
    if (P.l1 != H.l1 || P.l2 != H.l2 || P.l3 != H.l3 || P.o1 != H.o1 || P.o2 != H.o2 ||
        P.o3 != H.o3) {
      *why = "kernel path order disagrees with the host path enumeration";
      return false;
    }
    const int n2 = 2 * H.l2 + 1, n3 = 2 * H.l3 + 1;
    const std::vector<double>& C = p->cg[q];
    std::vector<char> covered(C.size(), 0);
    for (int e = P.nnz_begin; e < P.nnz_end; ++e) {
      const e3c::Entry& en = T.entry[e];
      const size_t idx = ((size_t)en.m1 * n2 + en.m2) * n3 + en.m3;
      coef[e] = C[idx];
      covered[idx] = 1;
    }
    for (size_t i = 0; i < C.size(); ++i) {
      if (C[i] != 0.0 && !covered[i]) {
        *why = "a nonzero CG entry lies outside the kernel's selection-rule pattern";
        return false;
      }
    }
  }
  // the kernels' compile-time values must equal the runtime tables (fp32 rounding)
  for (int e = 0; e < T.nnz; ++e) {
    const double d = std::fabs((double)ks->cg_values[e] - coef[e]);
    if (d > 1e-7 * std::fabs(coef[e]) + 1e-12) {
      *why = "compiled CG value " + std::to_string(e) + " disagrees with the plan's table";
      return false;
    }
  }
  p->ks = ks;
  p->kk = p->ordering == E3CONV_SENDER ? &ks->sender : &ks->receiver;
  return true;
}

}  // namespace

extern "C" {

const char* e3conv_status_string(e3conv_status st) {
  switch (st) {
    case E3CONV_OK: return "ok";
    case E3CONV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case E3CONV_ERR_PARSE: return "irreps parse error";
    case E3CONV_ERR_UNSUPPORTED: return "unsupported layout or dtype";
    case E3CONV_ERR_NO_PATH: return "output irrep reached by no path";
    case E3CONV_ERR_GRAPH: return "invalid graph";
    case E3CONV_ERR_WORKSPACE: return "workspace too small";
    case E3CONV_ERR_HIP: return "HIP runtime error";
    case E3CONV_ERR_INTERNAL: return "internal consistency error";
  }
  return "unknown status";
}

const char* e3conv_last_error_detail(void) { return g_last_error.c_str(); }

e3conv_status e3conv_plan(const char* irreps_in, int sh_lmax, const char* irreps_out,
                          float avg_num_neighbors, e3conv_plan_t* plan_out) {
  return e3conv_plan_ordered(irreps_in, sh_lmax, irreps_out, avg_num_neighbors, E3CONV_RECEIVER,
                             plan_out);
}

e3conv_status e3conv_plan_ordered(const char* irreps_in, int sh_lmax, const char* irreps_out,
                                  float avg_num_neighbors, e3conv_ordering ordering,
                                  e3conv_plan_t* plan_out) {
  if (!plan_out) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan_out is NULL");
  *plan_out = nullptr;
  if (ordering != E3CONV_RECEIVER && ordering != E3CONV_SENDER)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "ordering must be RECEIVER or SENDER");
  if (!irreps_in || !irreps_out) return fail(E3CONV_ERR_INVALID_ARGUMENT, "irreps string is NULL");
  if (sh_lmax < 0 || sh_lmax > 6) return fail(E3CONV_ERR_INVALID_ARGUMENT, "sh_lmax must be in 0..6");
  if (!(avg_num_neighbors > 0.0f) || !std::isfinite(avg_num_neighbors))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "avg_num_neighbors must be positive and finite");
  std::unique_ptr<e3conv_plan_s> p(new (std::nothrow) e3conv_plan_s());
  if (!p) return fail(E3CONV_ERR_INTERNAL, "out of host memory");
  std::string err;
  if (!e3c::parse_irreps(irreps_in, &p->xin, &err))
    return fail(E3CONV_ERR_PARSE, std::string("irreps_in: ") + err);
  if (!e3c::parse_irreps(irreps_out, &p->out, &err))
    return fail(E3CONV_ERR_PARSE, std::string("irreps_out: ") + err);
  const int C = p->xin[0].mul;
  if (C <= 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "multiplicity must be positive");
  for (const auto* list : {&p->xin, &p->out})
    for (const Irrep& b : *list) {
      if (b.mul != C)
        return fail(E3CONV_ERR_INVALID_ARGUMENT, "all blocks need the same multiplicity");
      if (b.l > 6) return fail(E3CONV_ERR_UNSUPPORTED, "irreps with l > 6 are not supported");
    }
  for (const auto* list : {&p->xin, &p->out})
    for (size_t i = 0; i < list->size(); ++i)
      for (size_t j = i + 1; j < list->size(); ++j)
        if ((*list)[i].l == (*list)[j].l && (*list)[i].parity == (*list)[j].parity)
          return fail(E3CONV_ERR_INVALID_ARGUMENT, "duplicate irreps in a block list");
  p->channels = C;
  p->lmax = sh_lmax;
  p->avg = avg_num_neighbors;
  p->ordering = ordering;
  for (const Irrep& b : p->xin) p->num_x += 2 * b.l + 1;
  for (const Irrep& b : p->out) p->num_out += 2 * b.l + 1;
  p->num_y = (sh_lmax + 1) * (sh_lmax + 1);
  p->paths = e3c::enumerate_paths(p->xin, sh_lmax, p->out);
  std::vector<char> reached(p->out.size(), 0);
  for (const HostPath& h : p->paths) reached[h.i3] = 1;
  for (size_t i = 0; i < reached.size(); ++i)
    if (!reached[i])
      return fail(E3CONV_ERR_NO_PATH, "output block " + std::to_string(p->out[i].l) +
                                          (p->out[i].parity > 0 ? "e" : "o") + " is reached by no path");
  if ((int)p->paths.size() > e3c::kMaxPaths)
    return fail(E3CONV_ERR_UNSUPPORTED, "too many paths");
  for (size_t q = 0; q < p->paths.size(); ++q) {
    const HostPath& h = p->paths[q];
    std::vector<double> cg;
    if (!e3c::real_cg(h.l1, h.l2, h.l3, &cg))
      return fail(E3CONV_ERR_INTERNAL, "real CG construction failed");
    const int n1 = 2 * h.l1 + 1, n2 = 2 * h.l2 + 1, n3 = 2 * h.l3 + 1;
    for (int a = 0; a < n1; ++a)
      for (int b = 0; b < n2; ++b)
        for (int c = 0; c < n3; ++c) {
          const double v = cg[((size_t)a * n2 + b) * n3 + c];
          if (v == 0.0) continue;
          p->ix.push_back(h.o1 + a);
          p->iy.push_back(h.o2 + b);
          p->ip.push_back((int)q);
          p->iout.push_back(h.o3 + c);
          p->val.push_back(v);
        }
    p->cg.push_back(std::move(cg));
  }
  std::string why;
  if (!bind_kernels(p.get(), &why) && !why.empty()) return fail(E3CONV_ERR_INTERNAL, why);
  *plan_out = p.release();
  return ok();
}

void e3conv_plan_destroy(e3conv_plan_t plan) { delete plan; }

e3conv_status e3conv_plan_shape(e3conv_plan_t p, int* channels, int* num_x, int* num_y,
                                int* num_paths, int* num_out) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (channels) *channels = p->channels;
  if (num_x) *num_x = p->num_x;
  if (num_y) *num_y = p->num_y;
  if (num_paths) *num_paths = (int)p->paths.size();
  if (num_out) *num_out = p->num_out;
  return ok();
}

e3conv_status e3conv_plan_paths(e3conv_plan_t p, int* l1, int* p1, int* l2, int* l3, int* p3,
                                int* o1, int* o2, int* o3) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  for (size_t q = 0; q < p->paths.size(); ++q) {
    const HostPath& h = p->paths[q];
    if (l1) l1[q] = h.l1;
    if (p1) p1[q] = h.p1;
    if (l2) l2[q] = h.l2;
    if (l3) l3[q] = h.l3;
    if (p3) p3[q] = h.p3;
    if (o1) o1[q] = h.o1;
    if (o2) o2[q] = h.o2;
    if (o3) o3[q] = h.o3;
  }
  return ok();
}

e3conv_status e3conv_plan_coefficients(e3conv_plan_t p, int* nnz, int* ix, int* iy, int* ip,
                                       int* iout, double* value) {
  if (!p || !nnz) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan or nnz is NULL");
  *nnz = (int)p->val.size();
  for (size_t q = 0; q < p->val.size(); ++q) {
    if (ix) ix[q] = p->ix[q];
    if (iy) iy[q] = p->iy[q];
    if (ip) ip[q] = p->ip[q];
    if (iout) iout[q] = p->iout[q];
    if (value) value[q] = p->val[q];
  }
  return ok();
}

e3conv_status e3conv_plan_ordering(e3conv_plan_t p, e3conv_ordering* ordering) {
  if (!p || !ordering) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan or ordering is NULL");
  *ordering = p->ordering;
  return ok();
}

e3conv_status e3conv_plan_supported(e3conv_plan_t p, int* fwd_f32, int* fwd_bf16, int* bwd_f32) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (fwd_f32) *fwd_f32 = p->kk && p->kk->n_fwd_f32 > 0;
  if (fwd_bf16) *fwd_bf16 = p->kk && p->kk->n_fwd_bf16 > 0;
  if (bwd_f32) *bwd_f32 = p->kk && p->kk->n_bwd_f32 > 0;
  return ok();
}

e3conv_status e3conv_plan_num_variants(e3conv_plan_t p, e3conv_dtype dt, int* nf, int* nb) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (dt != E3CONV_F32 && dt != E3CONV_BF16) return fail(E3CONV_ERR_INVALID_ARGUMENT, "bad dtype");
  if (nf) *nf = p->kk ? (dt == E3CONV_F32 ? p->kk->n_fwd_f32 : p->kk->n_fwd_bf16) : 0;
  if (nb) *nb = p->kk ? (dt == E3CONV_F32 ? p->kk->n_bwd_f32 : 0) : 0;
  return ok();
}

e3conv_status e3conv_plan_set_variant(e3conv_plan_t p, int fv, int bv) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!p->kk) return fail(E3CONV_ERR_UNSUPPORTED, "no kernels for this layout");
  const int maxf = p->kk->n_fwd_f32 > p->kk->n_fwd_bf16 ? p->kk->n_fwd_f32 : p->kk->n_fwd_bf16;
  if (fv < 0 || fv >= maxf || bv < 0 || bv >= (p->kk->n_bwd_f32 > 0 ? p->kk->n_bwd_f32 : 1))
    return fail(E3CONV_ERR_UNSUPPORTED, "unknown kernel variant");
  p->fwd_variant = fv;
  p->bwd_variant = bv;
  return ok();
}

static e3conv_status check_sizes(int64_t N, int64_t E, int channels, int width) {
  if (N < 0 || E < 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "negative size");
  if (E >= (int64_t)1 << 31 || N >= ((int64_t)1 << 31) - 1)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "sizes must fit int32 indices");
  if (N * (int64_t)width * channels >= (int64_t)1 << 31)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "node tensor exceeds 2^31 elements");
  return E3CONV_OK;
}

e3conv_status e3conv_forward(e3conv_plan_t p, e3conv_dtype dt, const void* x, const void* y,
                             const void* s, const int32_t* src, const int32_t* row_ptr,
                             const int32_t* order, int64_t N, int64_t E, float* out, void* stream) {
  return e3conv_forward_masked(p, dt, x, y, s, src, row_ptr, order, N, E, N, out, stream);
}

e3conv_status e3conv_forward_masked(e3conv_plan_t p, e3conv_dtype dt, const void* x, const void* y,
                                    const void* s, const int32_t* src, const int32_t* row_ptr,
                                    const int32_t* order, int64_t N, int64_t E,
                                    int64_t num_real_nodes, float* out, void* stream) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (dt != E3CONV_F32 && dt != E3CONV_BF16) return fail(E3CONV_ERR_INVALID_ARGUMENT, "bad dtype");
  e3conv_status st = check_sizes(N, E, p->channels, p->num_out > p->num_x ? p->num_out : p->num_x);
  if (st != E3CONV_OK) return st;
  if (num_real_nodes < 0 || num_real_nodes > N)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "num_real_nodes must be in [0, num_nodes]");
  if (N == 0) return ok();
  if (!out || !row_ptr || (E > 0 && (!x || !y || !s || !src)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (!p->kk) return fail(E3CONV_ERR_UNSUPPORTED, "no compiled kernel for this layout");
  const int n = dt == E3CONV_F32 ? p->kk->n_fwd_f32 : p->kk->n_fwd_bf16;
  if (n == 0) return fail(E3CONV_ERR_UNSUPPORTED, "no compiled kernel for this dtype");
  const e3c::FwdLauncher* L = dt == E3CONV_F32 ? p->kk->fwd_f32 : p->kk->fwd_bf16;
  const int v = p->fwd_variant < n ? p->fwd_variant : 0;
  e3c::FwdParams prm{x, y, s, src, row_ptr, order, out, (int)N, (int)E, 1.0f / p->avg,
                     (int)num_real_nodes};
  const hipError_t err = L[v](prm, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "forward launch");
  return ok();
}

e3conv_status e3conv_forward_linear(e3conv_plan_t p, e3conv_dtype dt, const void* x, const void* y,
                                    const void* s, const int32_t* src, const int32_t* row_ptr,
                                    const int32_t* order, int64_t N, int64_t E, float scale,
                                    const float* weights, float* out, void* stream) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (dt != E3CONV_F32 && dt != E3CONV_BF16) return fail(E3CONV_ERR_INVALID_ARGUMENT, "bad dtype");
  e3conv_status st = check_sizes(N, E, p->channels, p->num_out > p->num_x ? p->num_out : p->num_x);
  if (st != E3CONV_OK) return st;
  if (!std::isfinite(scale)) return fail(E3CONV_ERR_INVALID_ARGUMENT, "scale must be finite");
  const e3c::FwdLauncher L = !p->kk ? nullptr : (dt == E3CONV_F32 ? p->kk->fwd_lin_f32 : p->kk->fwd_lin_bf16);
  if (!L)
    return fail(E3CONV_ERR_UNSUPPORTED,
                "no fused output-linear kernel for this layout (call e3conv_forward, then e3conv_linear)");
  if (N == 0) return ok();
  if (!out || !row_ptr || !weights || (E > 0 && (!x || !y || !s || !src)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  e3c::FwdParams prm{x, y, s, src, row_ptr, order, out, (int)N, (int)E, 1.0f / p->avg, (int)N, weights,
                     (float)(scale / std::sqrt((double)p->channels) / p->avg)};
  const hipError_t err = L(prm, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "forward-linear launch");
  return ok();
}

e3conv_status e3conv_forward_pairs(e3conv_plan_t p, const float* x, const float* y, const float* s,
                                   const int32_t* src, const int32_t* row_ptr, const int32_t* pair_of,
                                   const int32_t* order, int64_t N, int64_t E, int64_t num_pairs,
                                   float* out, void* stream) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  e3conv_status st = check_sizes(N, E, p->channels, p->num_out > p->num_x ? p->num_out : p->num_x);
  if (st != E3CONV_OK) return st;
  if (num_pairs < 0 || num_pairs > E) return fail(E3CONV_ERR_INVALID_ARGUMENT, "num_pairs out of range");
  if (p->ordering != E3CONV_RECEIVER)
    return fail(E3CONV_ERR_UNSUPPORTED, "the pair-stored forward takes a RECEIVER plan");
  if (!p->kk || !p->kk->fwd_pairs_f32)
    return fail(E3CONV_ERR_UNSUPPORTED, "no compiled pair-stored forward for this layout");
  if (N == 0) return ok();
  if (!out || !row_ptr || (E > 0 && (!x || !y || !s || !src || !pair_of)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  e3c::FwdParams prm{x, y, s, src, row_ptr, order, out, (int)N, (int)E, 1.0f / p->avg, (int)N, nullptr,
                     0.0f, pair_of};
  const hipError_t err = p->kk->fwd_pairs_f32(prm, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "pair-stored forward launch");
  return ok();
}

e3conv_status e3conv_forward_radial(e3conv_plan_t p, const float* x, const float* y, const float* r,
                                    const float* w1, const float* w2, int32_t num_basis,
                                    int32_t hidden, float r_max, float sigma, const int32_t* src,
                                    const int32_t* row_ptr, const int32_t* order, int64_t N, int64_t E,
                                    int64_t num_real_nodes, float* out, void* stream) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  e3conv_status st = check_sizes(N, E, p->channels, p->num_out > p->num_x ? p->num_out : p->num_x);
  if (st != E3CONV_OK) return st;
  if (num_real_nodes < 0 || num_real_nodes > N)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "num_real_nodes must be in [0, num_nodes]");
  if (num_basis < 2 || num_basis > 8)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "num_basis must be in [2, 8]");
  if (hidden < 4 || hidden > 128 || hidden % 4 != 0)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "hidden must be a multiple of 4 in [4, 128]");
  if (!(r_max > 0.0f) || !(sigma > 0.0f))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "r_max and sigma must be positive");
  if (!p->kk || !p->kk->radial_f32)
    return fail(E3CONV_ERR_UNSUPPORTED, "no radial-scalar kernel for this layout and ordering");
  if (N == 0) return ok();
  if (!out || !row_ptr || !w1 || !w2 || (E > 0 && (!x || !y || !r || !src)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  e3c::RadialParams prm{x, y, r, w1, w2, src, row_ptr, order, out, (int)N, (int)E, 1.0f / p->avg,
                        (int)num_real_nodes, num_basis, hidden, r_max, sigma};
  const hipError_t err = p->kk->radial_f32(prm, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "radial forward launch");
  return ok();
}

e3conv_status e3conv_jvp(e3conv_plan_t p, e3conv_dtype dt, const void* x, const void* y,
                         const void* s, const void* dx, const void* dy, const void* ds,
                         const int32_t* src, const int32_t* row_ptr, const int32_t* order,
                         int64_t N, int64_t E, int64_t num_real_nodes, float* out, float* out_dot,
                         void* stream) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (dt != E3CONV_F32 && dt != E3CONV_BF16) return fail(E3CONV_ERR_INVALID_ARGUMENT, "bad dtype");
  e3conv_status st = check_sizes(N, E, p->channels, p->num_out > p->num_x ? p->num_out : p->num_x);
  if (st != E3CONV_OK) return st;
  if (num_real_nodes < 0 || num_real_nodes > N)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "num_real_nodes must be in [0, num_nodes]");
  if (N == 0) return ok();
  if (!out_dot || !row_ptr || (E > 0 && (!x || !y || !s || !dx || !dy || !ds || !src)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (!p->kk) return fail(E3CONV_ERR_UNSUPPORTED, "no compiled kernel for this layout");
  const e3c::JvpLauncher L = dt == E3CONV_F32 ? p->kk->jvp_f32 : p->kk->jvp_bf16;
  if (!L) return fail(E3CONV_ERR_UNSUPPORTED, "no compiled forward-mode kernel for this dtype");
  e3c::JvpParams prm{x, y, s, dx, dy, ds, src, row_ptr, order, out, out_dot,
                     (int)N, (int)E, 1.0f / p->avg, (int)num_real_nodes};
  const hipError_t err = L(prm, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "jvp launch");
  return ok();
}

e3conv_status e3conv_backward_workspace_size(e3conv_plan_t p, int64_t N, int64_t E, size_t* bytes) {
  if (!p || !bytes) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan or bytes is NULL");
  if (N < 0 || E < 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "negative size");
  *bytes = 0;
  return ok();
}

e3conv_status e3conv_backward(e3conv_plan_t p, e3conv_dtype dt, const void* x, const void* y,
                              const void* s, const int32_t* src, const int32_t* row_ptr,
                              const int32_t* order, int64_t N, int64_t E, const float* g,
                              float* gx, float* gy,
                              float* gs, void* workspace, size_t workspace_bytes, void* stream) {
  if (!gx && !gy && !gs) {
    if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
    return ok();
  }
  if (!gx || (E > 0 && (!gy || !gs)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "grad_x, grad_y and grad_s are all required");
  return e3conv_backward_ex(p, dt, x, y, s, src, row_ptr, order, N, E, N, g, gx, gy, gs, 0u,
                            workspace, workspace_bytes, stream);
}

e3conv_status e3conv_backward_ex(e3conv_plan_t p, e3conv_dtype dt, const void* x, const void* y,
                                 const void* s, const int32_t* src, const int32_t* row_ptr,
                                 const int32_t* order, int64_t N, int64_t E, int64_t num_real_nodes,
                                 const float* g, float* gx, float* gy, float* gs, unsigned flags,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (dt != E3CONV_F32) return fail(E3CONV_ERR_UNSUPPORTED, "the reverse pass is fp32 only");
  e3conv_status st = check_sizes(N, E, p->channels, p->num_out > p->num_x ? p->num_out : p->num_x);
  if (st != E3CONV_OK) return st;
  if (num_real_nodes < 0 || num_real_nodes > N)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "num_real_nodes must be in [0, num_nodes]");
  if (flags & ~(unsigned)(E3CONV_ACCUMULATE_GRAD_X | E3CONV_ACCUMULATE_GRAD_Y | E3CONV_ACCUMULATE_GRAD_S))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "unknown flag bits");
  if (!gx && !gy && !gs) return ok();
  if (N == 0) return ok();
  if (!g || !row_ptr || (E > 0 && (!x || !y || !s || !src)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (!p->kk || p->kk->n_bwd_f32 == 0)
    return fail(E3CONV_ERR_UNSUPPORTED, "no compiled reverse kernel for this layout");
  e3c::BwdParams prm{static_cast<const float*>(x), static_cast<const float*>(y),
                     static_cast<const float*>(s), src, row_ptr, order, g, gx, gy, gs, (int)N, (int)E,
                     1.0f / p->avg, (int)num_real_nodes, (int)flags};
  e3c::BwdLauncher L;
  if (flags == 0 && gx && gy && gs) {
    L = p->kk->bwd_f32[p->bwd_variant < p->kk->n_bwd_f32 ? p->bwd_variant : 0];
  } else {
    L = p->kk->bwd_f32_general;
    if (!L) return fail(E3CONV_ERR_UNSUPPORTED, "no general reverse kernel for this layout");
  }
  const hipError_t err = L(prm, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "backward launch");
  return ok();
}

e3conv_status e3conv_second_derivatives(e3conv_plan_t p, e3conv_dtype dt, const void* x,
                                        const void* y, const void* s, const int32_t* src,
                                        const int32_t* row_ptr, const int32_t* order, int64_t N,
                                        int64_t E, int64_t num_real_nodes, const float* g,
                                        const float* cx, const float* cy, const float* cs,
                                        float* dx, float* dy, float* ds, float* dg, void* stream) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (dt != E3CONV_F32) return fail(E3CONV_ERR_UNSUPPORTED, "second derivatives are fp32 only");
  if (N > 0 && (!g || !cx || !dx || !dg)) return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (E > 0 && (!cy || !cs || !dy || !ds)) return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  // L2 = <cx, grad_x> + <cy, grad_y> + <cs, grad_s> = <g, D conv(x, y, s)[cx, cy, cs]>.  The
  // convolution is trilinear, so each partial derivative is a reverse pass with one operand
  // replaced by its cotangent, and dL2/dg is the forward-mode derivative along (cx, cy, cs).
  e3conv_status st = e3conv_backward_ex(p, dt, cx, y, s, src, row_ptr, order, N, E, num_real_nodes,
                                        g, nullptr, dy, ds, 0u, nullptr, 0, stream);
  if (st != E3CONV_OK) return st;
  st = e3conv_backward_ex(p, dt, x, cy, s, src, row_ptr, order, N, E, num_real_nodes, g, dx, nullptr,
                          ds, E3CONV_ACCUMULATE_GRAD_S, nullptr, 0, stream);
  if (st != E3CONV_OK) return st;
  st = e3conv_backward_ex(p, dt, x, y, cs, src, row_ptr, order, N, E, num_real_nodes, g, dx, dy,
                          nullptr, E3CONV_ACCUMULATE_GRAD_X | E3CONV_ACCUMULATE_GRAD_Y, nullptr, 0,
                          stream);
  if (st != E3CONV_OK) return st;
  return e3conv_jvp(p, dt, x, y, s, cx, cy, cs, src, row_ptr, order, N, E, num_real_nodes, nullptr,
                    dg, stream);
}

e3conv_status e3conv_backward_pairs(e3conv_plan_t p, const float* x, const float* y, const float* s,
                                    const int32_t* src, const int32_t* dst, int64_t N, int64_t E,
                                    const float* g, float* gx, float* gy, float* gs, void* stream) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  e3conv_status st = check_sizes(N, E, p->channels, p->num_out > p->num_x ? p->num_out : p->num_x);
  if (st != E3CONV_OK) return st;
  if (E > 0 && N == 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "stored edges need nodes");
  if (N == 0) return ok();
  if (!g || !gx || (E > 0 && (!x || !y || !s || !src || !dst || !gy || !gs)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (p->ordering != E3CONV_RECEIVER)
    return fail(E3CONV_ERR_UNSUPPORTED, "the pair-stored reverse pass takes a RECEIVER plan");
  if (!p->kk || !p->kk->bwd_pairs_f32)
    return fail(E3CONV_ERR_UNSUPPORTED, "no compiled pair-stored reverse kernel for this layout");
  e3c::BwdParams prm{x, y, s, src, nullptr, nullptr, g, gx, gy, gs, (int)N, (int)E, 1.0f / p->avg,
                     (int)N, 0, 0, dst};
  const hipError_t err = p->kk->bwd_pairs_f32(prm, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "pair-stored backward launch");
  return ok();
}

// ------------------------------------------------------------- linear ---

namespace {

e3conv_status linear_setup(e3conv_plan_t p, int c_out, float scale, int64_t N, e3c::LinearGemm* g) {
  if (!p) return fail(E3CONV_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (c_out <= 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "channels_out must be positive");
  if (!std::isfinite(scale)) return fail(E3CONV_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (N < 0 || N >= ((int64_t)1 << 31) - 1) return fail(E3CONV_ERR_INVALID_ARGUMENT, "bad num_nodes");
  if (p->num_out > e3c::kMaxLinearComponents)
    return fail(E3CONV_ERR_UNSUPPORTED, "too many output components for the linear");
  const int64_t width = p->channels > c_out ? p->channels : c_out;
  if (N * p->num_out * width >= (int64_t)1 << 31)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "node tensor exceeds 2^31 elements");
  std::memset(g, 0, sizeof(*g));
  int o = 0;
  for (size_t k = 0; k < p->out.size(); ++k)
    for (int m = 0; m < 2 * p->out[k].l + 1; ++m) g->comp_block[o++] = (int)k;
  g->num_comp = p->num_out;
  g->alpha = scale / std::sqrt((float)p->channels);
  return E3CONV_OK;
}

// out = in W_k and grad_in = grad_out W_k^T: the row-streaming kernel when the
// weight block fits its LDS tiling (K, N <= 128), else the tiled kernel.
hipError_t linear_by_rows(const e3c::LinearGemm& g, hipStream_t s) {
  if (g.K <= 128 && g.N <= 128) return e3c::launch_linear_rows(g, s);
  return e3c::launch_linear_gemm(g, 1, s);
}

}  // namespace

e3conv_status e3conv_linear(e3conv_plan_t p, int c_out, float scale, const float* w, const float* in,
                            int64_t N, float* out, void* stream) {
  e3c::LinearGemm g;
  const e3conv_status st = linear_setup(p, c_out, scale, N, &g);
  if (st != E3CONV_OK) return st;
  if (N == 0) return ok();
  if (!w || !in || !out) return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  const long C = p->channels, NO = p->num_out;
  g.A = in;   g.a_i = NO * C;      g.a_k = 1;  g.a_comp = C;
  g.B = w;    g.b_k = c_out;       g.b_j = 1;  g.b_comp = 0;     g.b_block = C * c_out;
  g.C = out;  g.c_i = NO * c_out;  g.c_j = 1;  g.c_comp = c_out; g.c_block = 0;
  g.M = (int)N; g.N = c_out; g.K = (int)C; g.k_chunk = (int)C;
  const hipError_t err = linear_by_rows(g, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "linear launch");
  return ok();
}

e3conv_status e3conv_linear_backward(e3conv_plan_t p, int c_out, float scale, const float* w,
                                     const float* in, int64_t N, const float* grad_out,
                                     float* grad_in, float* grad_w, void* stream) {
  e3c::LinearGemm g;
  e3conv_status st = linear_setup(p, c_out, scale, N, &g);
  if (st != E3CONV_OK) return st;
  if (!grad_in && !grad_w) return ok();
  if (!grad_out || (grad_in && !w) || (grad_w && !in))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  const long C = p->channels, NO = p->num_out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (grad_in && N > 0) {
    e3c::LinearGemm a = g;
    a.A = grad_out; a.a_i = NO * c_out; a.a_k = 1;  a.a_comp = c_out;
    a.B = w;        a.b_k = 1;          a.b_j = c_out; a.b_comp = 0; a.b_block = C * c_out;
    a.C = grad_in;  a.c_i = NO * C;     a.c_j = 1;  a.c_comp = C;  a.c_block = 0;
    a.M = (int)N; a.N = (int)C; a.K = c_out; a.k_chunk = c_out;
    const hipError_t err = linear_by_rows(a, s);
    if (err != hipSuccess) return hip_fail(err, "linear backward launch");
  }
  if (grad_w) {
    hipError_t err = e3c::launch_fill_zero(grad_w, (size_t)p->out.size() * C * c_out, s);
    if (err != hipSuccess) return hip_fail(err, "fill launch");
    if (N > 0) {
      e3c::LinearGemm b = g;
      b.A = in;       b.a_i = 1;       b.a_k = NO * C;     b.a_comp = C;
      b.B = grad_out; b.b_k = NO * c_out; b.b_j = 1;    b.b_comp = c_out; b.b_block = 0;
      b.C = grad_w;   b.c_i = c_out;   b.c_j = 1;        b.c_comp = 0;  b.c_block = C * c_out;
      b.M = (int)C; b.N = c_out; b.K = (int)N;
      // split the node reduction so the grid has about 512 work-groups (more splits
      // multiply the atomic additions into grad_w)
      const long tiles = ((C + 127) / 128) * ((c_out + 127) / 128) * NO;   // 128 x 128 tiles
      long splits = (512 + tiles - 1) / tiles;
      const long max_splits = (N + 255) / 256;
      if (splits > max_splits) splits = max_splits;
      if (splits < 1) splits = 1;
      if (splits * NO > 65535) splits = 65535 / NO;
      long chunk = (N + splits - 1) / splits;
      chunk = (chunk + 31) / 32 * 32;
      splits = (N + chunk - 1) / chunk;
      b.k_chunk = (int)chunk;
      b.atomic = 1;
      err = e3c::launch_linear_gemm(b, (int)splits, s);
      if (err != hipSuccess) return hip_fail(err, "linear weight-gradient launch");
    }
  }
  return ok();
}

e3conv_status e3conv_csr_from_receivers(const int32_t* dst, int64_t E, int64_t N, int32_t* row_ptr,
                                        void* stream) {
  if (N < 0 || E < 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "negative size");
  if (E >= (int64_t)1 << 31 || N >= ((int64_t)1 << 31) - 1)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "sizes must fit int32 indices");
  if (!row_ptr || (E > 0 && !dst)) return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  const hipError_t err =
      e3c::launch_csr_from_receivers(dst, (int)E, (int)N, row_ptr, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "csr launch");
  return ok();
}

e3conv_status e3conv_receiver_order(const int32_t* row_ptr, const int32_t* src, int64_t N,
                                    int64_t E, int cluster, int32_t* order) {
  if (N < 0 || E < 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "negative size");
  if (E >= (int64_t)1 << 31 || N >= ((int64_t)1 << 31) - 1)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "sizes must fit int32 indices");
  if (cluster <= 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "cluster must be positive");
  if (N == 0) return ok();
  if (!row_ptr || !order || (E > 0 && !src)) return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL pointer");
  const e3conv_status st = e3conv_validate_graph(src, row_ptr, N, E, 0);
  if (st != E3CONV_OK) return st;
  e3c::receiver_order(row_ptr, src, (int)N, cluster, order);
  return ok();
}

e3conv_status e3conv_relabel_nodes(const int32_t* row_ptr, const int32_t* src, int64_t N, int64_t E,
                                   int cluster, int32_t* node_new, int32_t* edge_perm) {
  if (N < 0 || E < 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "negative size");
  if (E >= (int64_t)1 << 31 || N >= ((int64_t)1 << 31) - 1)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "sizes must fit int32 indices");
  if (cluster <= 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "cluster must be positive");
  if (N == 0) return E == 0 ? ok() : fail(E3CONV_ERR_GRAPH, "edges without nodes");
  if (!row_ptr || !node_new || (E > 0 && (!src || !edge_perm)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL pointer");
  const e3conv_status st = e3conv_validate_graph(src, row_ptr, N, E, 0);
  if (st != E3CONV_OK) return st;
  std::vector<int> order((size_t)N);
  e3c::receiver_order(row_ptr, src, (int)N, cluster, order.data());
  for (int i = 0; i < (int)N; ++i) node_new[order[i]] = i;
  // new receiver b' = node_new[b] takes the edges of old receiver order[b'], in
  // new-receiver order; within one receiver, stable by new sender
  int64_t k = 0;
  for (int nb = 0; nb < (int)N; ++nb) {
    const int b = order[nb];
    const int64_t k0 = k;
    for (int e = row_ptr[b]; e < row_ptr[b + 1]; ++e) edge_perm[k++] = e;
    std::stable_sort(edge_perm + k0, edge_perm + k,
                     [&](int32_t a, int32_t c) { return node_new[src[a]] < node_new[src[c]]; });
  }
  return ok();
}

e3conv_status e3conv_pair_layout(const int32_t* row_ptr, const int32_t* src, int64_t N, int64_t E,
                                 int cluster, int32_t* stored, int32_t* pair_of) {
  if (N < 0 || E < 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "negative size");
  if (E >= (int64_t)1 << 31 || N >= ((int64_t)1 << 31) - 1)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "sizes must fit int32 indices");
  if (cluster <= 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "cluster must be positive");
  if (E % 2 != 0) return fail(E3CONV_ERR_GRAPH, "a symmetric graph has an even number of edges");
  if (N == 0) return E == 0 ? ok() : fail(E3CONV_ERR_GRAPH, "edges without nodes");
  if (!row_ptr || (E > 0 && (!src || !stored || !pair_of)))
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL pointer");
  const e3conv_status st = e3conv_validate_graph(src, row_ptr, N, E, 0);
  if (st != E3CONV_OK) return st;
  std::vector<int> order(N), rank(N);
  e3c::receiver_order(row_ptr, src, (int)N, cluster, order.data());
  for (int i = 0; i < (int)N; ++i) rank[order[i]] = i;
  // one stored edge per pair: the edge into the endpoint that comes first in the order
  std::unordered_map<int64_t, int> slot;
  slot.reserve((size_t)E);
  int k = 0;
  for (int i = 0; i < (int)N; ++i) {
    const int b = order[i];
    for (int e = row_ptr[b]; e < row_ptr[b + 1]; ++e) {
      const int a = src[e];
      if (a == b) return fail(E3CONV_ERR_GRAPH, "self loop at edge " + std::to_string(e));
      if (rank[a] < rank[b]) continue;            // stored as the reverse edge, into a
      const int64_t key = (int64_t)std::min(a, b) * N + std::max(a, b);
      if (!slot.emplace(key, k).second)
        return fail(E3CONV_ERR_GRAPH, "duplicate edge " + std::to_string(e));
      if (k >= E / 2) return fail(E3CONV_ERR_GRAPH, "graph is not symmetric");
      stored[k++] = e;
    }
  }
  if (k != E / 2) return fail(E3CONV_ERR_GRAPH, "graph is not symmetric");
  std::vector<int> seen(k, 0);
  for (int b = 0; b < (int)N; ++b) {
    for (int e = row_ptr[b]; e < row_ptr[b + 1]; ++e) {
      const int a = src[e];
      const auto it = slot.find((int64_t)std::min(a, b) * N + std::max(a, b));
      if (it == slot.end() || ++seen[it->second] > 2)
        return fail(E3CONV_ERR_GRAPH, "graph is not symmetric at edge " + std::to_string(e));
      pair_of[e] = stored[it->second] == e ? it->second : ~it->second;
    }
  }
  return ok();
}

e3conv_status e3conv_stream_reference(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || bytes % 16 != 0) return fail(E3CONV_ERR_INVALID_ARGUMENT, "src NULL or bytes not a multiple of 16");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return fail(E3CONV_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  const hipError_t err = e3c::launch_stream(src, dst, bytes, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "stream launch");
  return ok();
}

}  // extern "C"

// C ABI of libgptq: argument validation, workspace carving, launch order,
// kernel timing. Every step of the computation runs in the HIP kernels of
// the sibling .hip files; this file only sequences them on the caller's
// stream. Declarations and the contract are in include/gptq.h.
#include "../../include/gptq.h"
#include "common.h"

#include <cstddef>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

using namespace gq;

namespace {

thread_local std::string g_err;

gptq_status fail(gptq_status st, const char* msg) {
  g_err = msg;
  return st;
}

gptq_status hip_fail(hipError_t e, const char* where) {
  g_err = std::string(where) + ": " + hipGetErrorString(e);
  return GPTQ_EHIP;
}

#define HIP_TRY(expr, where)                   \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// ---------------------------------------------------------------- timing
struct ProfRec {
  int cls;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records a start event on construction and a stop event on destruction
// when timing is enabled.
class Timed {
 public:
  Timed(int cls, hipStream_t s) : cls_(cls), s_(s) {
    if (!g_prof_on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    a_ = prof_event();
    b_ = prof_event();
    if (a_ && b_) hipEventRecord(a_, s_);
  }
  ~Timed() {
    if (!a_ || !b_) return;
    hipEventRecord(b_, s_);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_recs.push_back({cls_, a_, b_});
  }

 private:
  int cls_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};

// ---------------------------------------------------------------- workspace
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  }
};

// Columns per super-block of the two-level lazy batch: a multiple of the
// block width B, and of the group size when groups span several blocks, so
// that no group straddles two super-blocks (its statistics are taken from
// values that have received every earlier column's update).
int64_t super_width(const gptq_params* p) {
  const int64_t B = p->block, g = p->group;
  if (g <= B) return 512;                  // 512 is a multiple of B = 32, 64, 128
  return g <= 512 ? g * (512 / g) : g;     // g % B == 0
}

// The split-bf16 far-field update needs 8-element aligned rows and column
// origins; otherwise every block applies its own fp32 update to all later
// columns.
bool use_two_level(int64_t n, const gptq_params* p) { return n % 8 == 0 && super_width(p) % 8 == 0; }

struct QLayout {
  size_t status, lam, diag, perm, invperm, A, X, Wf, E, Ehi, Elo, Uhi, Ulo, codes, loss, total;
};

QLayout q_layout(int64_t d_out, int64_t n, const gptq_params* p) {
  QLayout L{};
  Carver c;
  const bool two = d_out > 0 && use_two_level(n, p);
  const int64_t ew = two ? super_width(p) : p->block;
  L.status = c.take(sizeof(DevStatus));
  L.lam = c.take(sizeof(double));
  L.diag = c.take(sizeof(float) * n);
  L.perm = c.take(sizeof(int32_t) * n);
  L.invperm = c.take(sizeof(int32_t) * n);
  L.A = c.take(sizeof(float) * n * n);
  L.X = c.take(sizeof(float) * n * n);
  L.Wf = c.take(sizeof(float) * d_out * n);
  L.E = c.take(sizeof(float) * d_out * ew);
  L.Ehi = c.take(two ? sizeof(uint16_t) * d_out * ew : 0);
  L.Elo = c.take(two ? sizeof(uint16_t) * d_out * ew : 0);
  L.Uhi = c.take(two ? sizeof(uint16_t) * n * n : 0);
  L.Ulo = c.take(two ? sizeof(uint16_t) * n * n : 0);
  L.codes = c.take((size_t)d_out * p->n_quant);
  L.loss = c.take(sizeof(float) * d_out);
  L.total = c.off;
  return L;
}

// The parameter block grows at its end; fields past a caller's struct_size
// take their defaults.
constexpr size_t kParamsMin = offsetof(gptq_params, sym);
int params_sym(const gptq_params* p) {
  return p->struct_size >= offsetof(gptq_params, sym) + sizeof(int32_t) ? p->sym : 0;
}

gptq_status check_params(int64_t d_out, int64_t n, const gptq_params* p) {
  if (!p) return fail(GPTQ_EINVAL, "params is NULL");
  if (p->struct_size < kParamsMin) return fail(GPTQ_EINVAL, "params.struct_size too small");
  if (d_out < 0 || n < 1) return fail(GPTQ_EINVAL, "need d_out >= 0 and n >= 1");
  if (n > (int64_t)1 << 30 || d_out > (int64_t)1 << 30) return fail(GPTQ_EINVAL, "dimension too large");
  if (p->bits < 2 || p->bits > 4) return fail(GPTQ_EINVAL, "bits must be 2, 3 or 4");
  if (p->block != 32 && p->block != 64 && p->block != 128)
    return fail(GPTQ_EINVAL, "block must be 32, 64 or 128");
  if (p->n_quant < 1 || p->n_quant > n) return fail(GPTQ_EINVAL, "n_quant must be in [1, n]");
  if (p->group < 8) return fail(GPTQ_EINVAL, "group must be >= 8");
  if (p->n_quant % p->group != 0) return fail(GPTQ_EINVAL, "group must divide n_quant");
  if (!(p->group % p->block == 0 || p->block % p->group == 0))
    return fail(GPTQ_EINVAL, "group and block must nest (one divides the other)");
  if (!(p->damp >= 0.f) || !std::isfinite(p->damp)) return fail(GPTQ_EINVAL, "damp must be finite and >= 0");
  if (p->act_order != 0 && p->act_order != 1) return fail(GPTQ_EINVAL, "act_order must be 0 or 1");
  const int sym = params_sym(p);
  if (sym != 0 && sym != 1) return fail(GPTQ_EINVAL, "sym must be 0 or 1");
  return GPTQ_OK;
}

// gptq_factor_hinv only uses n, damp, act_order and n_quant.
gptq_status check_factor_params(int64_t n, const gptq_params* p) {
  if (!p) return fail(GPTQ_EINVAL, "params is NULL");
  if (p->struct_size < kParamsMin) return fail(GPTQ_EINVAL, "params.struct_size too small");
  if (n < 1 || n > (int64_t)1 << 30) return fail(GPTQ_EINVAL, "need 1 <= n <= 2^30");
  if (p->n_quant < 1 || p->n_quant > n) return fail(GPTQ_EINVAL, "n_quant must be in [1, n]");
  if (!(p->damp >= 0.f) || !std::isfinite(p->damp)) return fail(GPTQ_EINVAL, "damp must be finite and >= 0");
  if (p->act_order != 0 && p->act_order != 1) return fail(GPTQ_EINVAL, "act_order must be 0 or 1");
  return GPTQ_OK;
}

gptq_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return GPTQ_OK;
  if (!ws) return fail(GPTQ_EWORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws % 256 != 0) return fail(GPTQ_EWORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(GPTQ_EWORKSPACE, "workspace too small");
  return GPTQ_OK;
}

// ---------------------------------------------------------------- factorisation
// Right-looking Cholesky of the flipped matrix A with the inverse X = L^{-1}
// carried along (see factor.hip): three launches per 64-column panel.
hipError_t factor_panels(hipStream_t s, float* A, float* X, int64_t n, const int32_t* perm,
                         DevStatus* st) {
  hipError_t e;
  // ---- phase 1: Cholesky, leaves write D = L11^{-1} into X's diagonal
  if ((e = launch_leaf(s, A, X, n, 0, std::min<int64_t>(kLeaf, n), perm, st)) != hipSuccess) return e;
  for (int64_t k0 = 0; k0 < n; k0 += kLeaf) {
    const int64_t m = std::min<int64_t>(kLeaf, n - k0);
    const int64_t k1 = k0 + m, r = n - k1;
    if (r == 0) break;
    const float* D = X + k0 * n + k0;    // L11^{-1}, lower
    float* L21 = A + k1 * n + k0;
    // L21 = A21 D^T in place (m == 64 whenever rows remain below the panel)
    if ((e = launch_panel_solve(s, L21, D, n, r)) != hipSuccess) return e;
    // One launch: the next diagonal block (m2 rows) is updated and factored
    // by its own workgroup while the rest runs
    //   A[k1+m2:, k1:] -= L21[m2:] L21^T   (lower, i.e. j <= i + m2)
    const int64_t m2 = std::min<int64_t>(kLeaf, r);
    SlabArgs g3{};
    g3.M = r - m2; g3.N = r; g3.K = m;
    g3.A = L21 + m2 * n; g3.lda = n;
    g3.B = L21; g3.ldb = n; g3.tb = 1;
    g3.C = A + (k1 + m2) * n + k1; g3.ldc = n;
    g3.alpha = -1.f; g3.beta = 1.f;
    g3.lower_only = 1; g3.lower_off = m2;
    LeafTask lt{L21, A, X, n, k1, (int)m2, (int)m, perm, st};
    if ((e = launch_slab_leaf(s, g3, lt)) != hipSuccess) return e;
  }
  // ---- phase 2: off-diagonal blocks of X = L^{-1}
  for (int64_t h = kLeaf; h < n; h *= 2) {
    const int64_t full = n / (2 * h);                        // pairs whose j block is complete
    const int64_t bp_last = full * 2 * h + h;                // j-block start of a partial pair
    const int64_t hj_last = bp_last < n ? n - bp_last : 0;   // its rows (0: none)
    const int64_t step = 2 * h * (n + 1);
    auto gemms = [&](int64_t ap, int64_t hj, int batch, GemmArgs& g1, GemmArgs& g2) {
      const int64_t bp = ap + h;
      // g1: T^T (h x hj) = X_ii^T L_ji^T, into A[ap:ap+h, bp:bp+hj] (upper, free)
      g1 = GemmArgs{};
      g1.M = h; g1.N = hj; g1.K = h;
      g1.A = X + ap * n + ap; g1.lda = n; g1.ta = 1;
      g1.B = A + bp * n + ap; g1.ldb = n; g1.tb = 1;
      g1.C = A + ap * n + bp; g1.ldc = n;
      g1.alpha = 1.f; g1.beta = 0.f; g1.kmode = 4;
      g1.batch = batch; g1.sA = step; g1.sB = step; g1.sC = step;
      // g2: X_ji (hj x h) = -X_jj T
      g2 = GemmArgs{};
      g2.M = hj; g2.N = h; g2.K = hj;
      g2.A = X + bp * n + bp; g2.lda = n; g2.ta = 0;
      g2.B = A + ap * n + bp; g2.ldb = n; g2.tb = 1;
      g2.C = X + bp * n + ap; g2.ldc = n;
      g2.alpha = -1.f; g2.beta = 0.f; g2.kmode = 3;
      g2.batch = batch; g2.sA = step; g2.sB = step; g2.sC = step;
    };
    GemmArgs f1{}, f2{}, p1{}, p2{};
    if (full > 0) gemms(0, h, (int)full, f1, f2);
    if (hj_last > 0) gemms(full * 2 * h, hj_last, 1, p1, p2);
    const GemmArgs* first1 = full > 0 ? &f1 : &p1;
    const GemmArgs* second1 = (full > 0 && hj_last > 0) ? &p1 : nullptr;
    const GemmArgs* first2 = full > 0 ? &f2 : &p2;
    const GemmArgs* second2 = (full > 0 && hj_last > 0) ? &p2 : nullptr;
    if ((e = launch_gemm_pair(s, *first1, second1)) != hipSuccess) return e;
    if ((e = launch_gemm_pair(s, *first2, second2)) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Steps 2-3 shared by quantize_layer and factor_hinv. On return (enqueued)
// the upper factor U is in the A buffer (processing order).
gptq_status enqueue_factor(hipStream_t s, const float* H, int64_t n, const gptq_params* p,
                           char* ws, const QLayout& L, uint16_t* Uhi = nullptr, uint16_t* Ulo = nullptr) {
  DevStatus* st = reinterpret_cast<DevStatus*>(ws + L.status);
  double* lam = reinterpret_cast<double*>(ws + L.lam);
  float* diag = reinterpret_cast<float*>(ws + L.diag);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  int32_t* invperm = reinterpret_cast<int32_t*>(ws + L.invperm);
  float* A = reinterpret_cast<float*>(ws + L.A);
  float* X = reinterpret_cast<float*>(ws + L.X);
  {
    HIP_TRY(launch_status_init(s, st), "status init");
    HIP_TRY(launch_fill_f32(s, X, (size_t)n * n, 0.f), "fill");
    HIP_TRY(launch_prep_diag(s, H, n, diag, lam, p->damp, st), "prep diag");
    HIP_TRY(launch_order(s, diag, n, p->n_quant, p->act_order, perm, invperm), "order");
    // the processing order is the identity without act-order
    HIP_TRY(launch_build_flipped(s, H, n, p->act_order ? perm : nullptr, diag, lam, A, st), "build");
  }
  HIP_TRY(factor_panels(s, A, X, n, perm, st), "factor");
  HIP_TRY(launch_rotate(s, X, A, n, Uhi, Ulo), "rotate");
  return GPTQ_OK;
}

gptq_status read_status(hipStream_t s, const DevStatus* st, const int32_t* perm, int64_t* fail_col) {
  DevStatus h{};
  HIP_TRY(hipMemcpyAsync(&h, st, sizeof(h), hipMemcpyDeviceToHost, s), "status copy");
  HIP_TRY(hipStreamSynchronize(s), "synchronize");
  (void)perm;
  if (h.flags == 0) return GPTQ_OK;
  if (fail_col) *fail_col = (h.col == ~0ull) ? -1 : (int64_t)h.col;
  if (h.flags & kNonFinite) return fail(GPTQ_ENONFINITE, "non-finite value in W or H");
  return fail(GPTQ_ENOTPD, "damped Hessian is not positive definite");
}

}  // namespace

extern "C" {

const char* gptq_status_string(int status) {
  switch (status) {
    case GPTQ_OK: return "ok";
    case GPTQ_EINVAL: return "invalid argument";
    case GPTQ_ENOTPD: return "damped Hessian not positive definite";
    case GPTQ_ENONFINITE: return "non-finite input";
    case GPTQ_EHIP: return "HIP error";
    case GPTQ_EWORKSPACE: return "workspace missing, misaligned or too small";
    default: return "unknown status";
  }
}

const char* gptq_last_error(void) { return g_err.c_str(); }

gptq_status gptq_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_recs) {
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  g_prof_on = enable != 0;
  return GPTQ_OK;
}

gptq_status gptq_profile_collect(double* ms, int64_t* count) {
  if (!ms || !count) return fail(GPTQ_EINVAL, "NULL output");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (int c = 0; c < GPTQ_PROF_NCLASSES; ++c) {
    ms[c] = 0.0;
    count[c] = 0;
  }
  for (auto& r : g_prof_recs) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "event sync");
    float t = 0.f;
    e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "event elapsed");
    ms[r.cls] += t;
    count[r.cls] += 1;
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  return GPTQ_OK;
}

gptq_status gptq_hessian_workspace_bytes(int64_t T, int64_t n, gptq_dtype xdt, size_t* bytes) {
  if (!bytes) return fail(GPTQ_EINVAL, "bytes is NULL");
  if (T < 0 || n < 1 || n > ((int64_t)1 << 30)) return fail(GPTQ_EINVAL, "need T >= 0, n >= 1");
  if (xdt != GPTQ_BF16 && xdt != GPTQ_F32) return fail(GPTQ_EINVAL, "bad dtype");
  if (T == 0) {
    *bytes = 0;
    return GPTQ_OK;
  }
  const int sp = hessian_splits(T, n);
  *bytes = (size_t)sp * n * n * sizeof(float);
  return GPTQ_OK;
}

gptq_status gptq_accumulate_hessian(void* stream, const void* X, gptq_dtype xdt, int64_t T, int64_t n,
                                    int64_t ldx, float* H, int zero_first, void* workspace,
                                    size_t workspace_bytes) {
  hipStream_t s = (hipStream_t)stream;
  size_t need = 0;
  gptq_status st = gptq_hessian_workspace_bytes(T, n, xdt, &need);
  if (st != GPTQ_OK) return st;
  if (!H) return fail(GPTQ_EINVAL, "H is NULL");
  if (T > 0 && !X) return fail(GPTQ_EINVAL, "X is NULL");
  if (ldx < n) return fail(GPTQ_EINVAL, "ldx < n");
  if ((st = check_ws(workspace, workspace_bytes, need)) != GPTQ_OK) return st;
  if (T == 0) {
    if (zero_first) HIP_TRY(launch_fill_f32(s, H, (size_t)n * n, 0.f), "fill");
    return GPTQ_OK;
  }
  const int sp = hessian_splits(T, n);
  float* part = reinterpret_cast<float*>(workspace);
  {
    Timed t(GPTQ_PROF_HESSIAN_SYRK, s);
    if (xdt == GPTQ_BF16)
      HIP_TRY(launch_hessian_partials_bf16(s, reinterpret_cast<const uint16_t*>(X), T, n, ldx, part, sp),
              "hessian partials");
    else
      HIP_TRY(launch_hessian_partials_f32(s, reinterpret_cast<const float*>(X), T, n, ldx, part, sp),
              "hessian partials");
  }
  {
    Timed t(GPTQ_PROF_HESSIAN_REDUCE, s);
    HIP_TRY(launch_hessian_reduce(s, part, sp, n, H, zero_first), "hessian reduce");
  }
  return GPTQ_OK;
}

gptq_status gptq_workspace_bytes(int64_t d_out, int64_t n, const gptq_params* p, size_t* bytes) {
  if (!bytes) return fail(GPTQ_EINVAL, "bytes is NULL");
  gptq_status st = d_out == 0 ? check_factor_params(n, p) : check_params(d_out, n, p);
  if (st != GPTQ_OK) return st;
  *bytes = q_layout(d_out, n, p).total;
  return GPTQ_OK;
}

gptq_status gptq_factor_hinv(void* stream, const float* H, int64_t n, const gptq_params* p,
                             void* workspace, size_t workspace_bytes, float* U_out, int32_t* perm_out,
                             int64_t* fail_col) {
  hipStream_t s = (hipStream_t)stream;
  gptq_status st = check_factor_params(n, p);
  if (st != GPTQ_OK) return st;
  if (!H || !U_out) return fail(GPTQ_EINVAL, "H or U_out is NULL");
  const QLayout L = q_layout(0, n, p);
  if ((st = check_ws(workspace, workspace_bytes, L.total)) != GPTQ_OK) return st;
  if (fail_col) *fail_col = -1;
  char* ws = reinterpret_cast<char*>(workspace);
  if ((st = enqueue_factor(s, H, n, p, ws, L)) != GPTQ_OK) return st;
  HIP_TRY(hipMemcpyAsync(U_out, ws + L.A, sizeof(float) * n * n, hipMemcpyDeviceToDevice, s), "copy U");
  if (perm_out)
    HIP_TRY(hipMemcpyAsync(perm_out, ws + L.perm, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, s),
            "copy perm");
  return read_status(s, reinterpret_cast<DevStatus*>(ws + L.status), nullptr, fail_col);
}

gptq_status gptq_quantize_layer(void* stream, const void* W, gptq_dtype wdt, int64_t d_out, int64_t n,
                                int64_t ldw, const float* H, const gptq_params* p, void* workspace,
                                size_t workspace_bytes, const gptq_outputs* out, int64_t* fail_col) {
  hipStream_t s = (hipStream_t)stream;
  gptq_status st = check_params(d_out, n, p);
  if (st != GPTQ_OK) return st;
  if (wdt != GPTQ_BF16 && wdt != GPTQ_F32) return fail(GPTQ_EINVAL, "bad dtype");
  if (!out) return fail(GPTQ_EINVAL, "outputs is NULL");
  if (!H) return fail(GPTQ_EINVAL, "H is NULL");
  if (d_out == 0) return GPTQ_OK;
  if (!W) return fail(GPTQ_EINVAL, "W is NULL");
  if (ldw < n) return fail(GPTQ_EINVAL, "ldw < n");
  if (!out->scales || !out->zeros) return fail(GPTQ_EINVAL, "scales and zeros are required");
  const QLayout L = q_layout(d_out, n, p);
  if ((st = check_ws(workspace, workspace_bytes, L.total)) != GPTQ_OK) return st;
  if (fail_col) *fail_col = -1;

  char* ws = reinterpret_cast<char*>(workspace);
  DevStatus* dst = reinterpret_cast<DevStatus*>(ws + L.status);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  {
  Timed whole(GPTQ_PROF_QUANTIZE, s);
  int32_t* invperm = reinterpret_cast<int32_t*>(ws + L.invperm);
  float* U = reinterpret_cast<float*>(ws + L.A);
  // Without act-order the processing order is the identity, so the working
  // copy can live in w_hat itself: it ends holding the dequantised weights
  // (and the updated unquantised columns) and needs no final copy.
  const bool in_place = !p->act_order && out->w_hat != nullptr;
  float* Wf = in_place ? out->w_hat : reinterpret_cast<float*>(ws + L.Wf);
  float* E = reinterpret_cast<float*>(ws + L.E);
  uint8_t* codes = reinterpret_cast<uint8_t*>(ws + L.codes);
  float* loss = out->row_loss ? out->row_loss : reinterpret_cast<float*>(ws + L.loss);

  const int64_t nq = p->n_quant;
  const int B = p->block;
  const bool two = use_two_level(n, p);
  const int64_t sw = two ? super_width(p) : B;   // columns per super-block; E's row pitch
  uint16_t* Ehi = reinterpret_cast<uint16_t*>(ws + L.Ehi);
  uint16_t* Elo = reinterpret_cast<uint16_t*>(ws + L.Elo);
  uint16_t* Uhi = reinterpret_cast<uint16_t*>(ws + L.Uhi);
  uint16_t* Ulo = reinterpret_cast<uint16_t*>(ws + L.Ulo);
  // the far field's split-bf16 operands are written by the kernels that
  // produce U (the final rotation) and E (the sweep)
  if ((st = enqueue_factor(s, H, n, p, ws, L, two ? Uhi : nullptr, two ? Ulo : nullptr)) != GPTQ_OK) return st;
  HIP_TRY(launch_w_prep(s, W, wdt == GPTQ_BF16, d_out, n, ldw, p->act_order ? perm : nullptr, Wf, dst),
          "w prep");
  HIP_TRY(launch_fill_f32(s, loss, (size_t)d_out, 0.f), "fill");
  // Two-level lazy batch. Inside a super-block [s0, s1) each block updates
  // the super-block's later columns at once (fp32, K = B); when the
  // super-block is done, all of its errors update the columns right of it
  // in one split-bf16 product (K = s1 - s0). Without the split path the
  // super-block is the block itself and the far field is fp32. With B = 128,
  // whole blocks and groups inside a block, the in-super-block update is
  // taken left-looking by the sweep kernel itself (each block first applies
  // the errors of the super-block's earlier blocks to its own columns).
  const bool fused = two && B == 128 && p->group <= B && nq % B == 0 && sw == 512;
  for (int64_t s0 = 0; s0 < nq; s0 += sw) {
    const int64_t s1 = std::min<int64_t>(s0 + sw, nq);
    for (int64_t i0 = s0; i0 < s1; i0 += B) {
      const int64_t nc = std::min<int64_t>(B, s1 - i0);
      float* Eb = E + (i0 - s0);
      SweepArgs a{};
      a.Wf = Wf; a.ldw = n; a.U = U; a.ldu = n; a.d_out = d_out; a.i0 = i0; a.ncols = nc;
      a.block = B; a.group = p->group; a.bits = p->bits; a.sym = params_sym(p);
      a.gbase = i0 / p->group;
      a.gshift = 31;
      if (p->group < B)
        for (int sh = 0; sh < 31; ++sh)
          if ((1 << sh) == p->group) a.gshift = sh;
      a.scales = out->scales; a.zeros = out->zeros; a.ngroups = nq / p->group;
      a.codes = codes; a.n_quant = nq; a.E = Eb; a.lde = sw; a.row_loss = loss; a.st = dst;
      a.Esb = E; a.kb = fused ? i0 - s0 : 0;
      a.Ehi = two && s1 < n ? Ehi + (i0 - s0) : nullptr;
      a.Elo = two && s1 < n ? Elo + (i0 - s0) : nullptr;
      HIP_TRY(launch_sweep(s, a), "sweep");
      const int64_t i1 = i0 + nc;
      const int64_t near_end = two ? s1 : n;
      if (!fused && i1 < near_end) {
        SlabArgs g{};
        g.M = d_out; g.N = near_end - i1; g.K = nc;
        g.A = Eb; g.lda = sw;
        g.B = U + i0 * n + i1; g.ldb = n; g.tb = 0;
        g.C = Wf + i1; g.ldc = n;
        g.alpha = -1.f; g.beta = 1.f;
        HIP_TRY(launch_slab(s, g), "near-field update");
      }
    }
    if (two && s1 < n) {
      TrailArgs t{};
      t.M = d_out; t.N = n - s1; t.K = s1 - s0;
      t.Ahi = Ehi; t.Alo = Elo; t.lda = sw;
      t.Bhi = Uhi + s0 * n + s1; t.Blo = Ulo + s0 * n + s1; t.ldb = n;
      t.C = Wf + s1; t.ldc = n;
      HIP_TRY(launch_trail_x3(s, t), "far-field update");
    }
  }
  HIP_TRY(launch_finish(s, Wf, codes, invperm, d_out, n, nq, p->group, in_place ? nullptr : out->w_hat,
                        out->codes, out->g_idx),
          "finish");
  // the processing order is the identity without act-order
  if (out->qweight)
    HIP_TRY(launch_pack(s, codes, nq, p->act_order ? invperm : nullptr, d_out, nq, p->bits, out->qweight),
            "pack");
  }
  return read_status(s, dst, perm, fail_col);
}

gptq_status gptq_pack_codes(void* stream, const uint8_t* codes, int64_t d_out, int64_t n_quant,
                            int32_t bits, uint32_t* qweight) {
  if (bits < 2 || bits > 4) return fail(GPTQ_EINVAL, "bits must be 2, 3 or 4");
  if (d_out < 0 || n_quant < 0) return fail(GPTQ_EINVAL, "negative size");
  if (d_out * n_quant > 0 && (!codes || !qweight)) return fail(GPTQ_EINVAL, "NULL pointer");
  HIP_TRY(launch_pack((hipStream_t)stream, codes, n_quant, nullptr, d_out, n_quant, bits, qweight), "pack");
  return GPTQ_OK;
}

gptq_status gptq_unpack_codes(void* stream, const uint32_t* qweight, int64_t d_out, int64_t n_quant,
                              int32_t bits, uint8_t* codes) {
  if (bits < 2 || bits > 4) return fail(GPTQ_EINVAL, "bits must be 2, 3 or 4");
  if (d_out < 0 || n_quant < 0) return fail(GPTQ_EINVAL, "negative size");
  if (d_out * n_quant > 0 && (!codes || !qweight)) return fail(GPTQ_EINVAL, "NULL pointer");
  HIP_TRY(launch_unpack((hipStream_t)stream, qweight, d_out, n_quant, bits, codes), "unpack");
  return GPTQ_OK;
}

// ---------------------------------------------------------------- inference
static gptq_status dq_check(int64_t M, int64_t n, int64_t d_out, int32_t bits, int32_t group) {
  if (bits < 2 || bits > 4) return fail(GPTQ_EINVAL, "bits must be 2, 3 or 4");
  if (M < 0 || n < 0 || d_out < 0) return fail(GPTQ_EINVAL, "negative size");
  if (group <= 0 || group % 32 != 0) return fail(GPTQ_EINVAL, "group must be a positive multiple of 32");
  if (n % group != 0) return fail(GPTQ_EINVAL, "group must divide n");
  return GPTQ_OK;
}

// bytes of the gathered activations (permuted product), then the partials
static size_t dq_xp_bytes(int64_t M, int64_t n, int permuted) {
  return permuted ? ((size_t)M * n * sizeof(uint16_t) + 255) / 256 * 256 : 0;
}

gptq_status gptq_dequant_matmul_workspace_bytes(int64_t M, int64_t n, int64_t d_out, int32_t bits,
                                                int32_t group, int32_t permuted, size_t* bytes) {
  if (!bytes) return fail(GPTQ_EINVAL, "NULL pointer");
  const gptq_status st = dq_check(M, n, d_out, bits, group);
  if (st != GPTQ_OK) return st;
  const DqPlan p = dequant_mm_plan(M, n, d_out, bits, group);
  *bytes = dq_xp_bytes(M, n, permuted) + (p.part_bytes + 255) / 256 * 256;
  return GPTQ_OK;
}

gptq_status gptq_repack_act_order_workspace_bytes(int64_t d_out, int64_t n, size_t* bytes) {
  if (!bytes) return fail(GPTQ_EINVAL, "NULL pointer");
  if (d_out < 0 || n < 0) return fail(GPTQ_EINVAL, "negative size");
  *bytes = ((size_t)d_out * n + 255) / 256 * 256;
  return GPTQ_OK;
}

gptq_status gptq_repack_act_order(void* stream, const uint32_t* qweight, const int32_t* g_idx, int64_t d_out,
                                  int64_t n, int32_t bits, int32_t group, uint32_t* qweight_out,
                                  int32_t* perm_out, void* workspace, size_t ws_bytes) {
  gptq_status st = dq_check(1, n, d_out, bits, group);
  if (st != GPTQ_OK) return st;
  if (n == 0) return GPTQ_OK;
  if (!g_idx || !perm_out) return fail(GPTQ_EINVAL, "NULL pointer");
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(launch_fill_f32(s, reinterpret_cast<float*>(perm_out), (size_t)n, 0.f), "fill");   // int32 zeros
  HIP_TRY(launch_group_order(s, g_idx, n, group, perm_out), "group order");
  if (d_out == 0) return GPTQ_OK;
  if (!qweight || !qweight_out) return fail(GPTQ_EINVAL, "NULL pointer");
  size_t need = 0;
  gptq_repack_act_order_workspace_bytes(d_out, n, &need);
  if ((st = check_ws(workspace, ws_bytes, need)) != GPTQ_OK) return st;
  uint8_t* codes = static_cast<uint8_t*>(workspace);
  HIP_TRY(launch_unpack(s, qweight, d_out, n, bits, codes), "unpack");
  HIP_TRY(launch_pack(s, codes, n, perm_out, d_out, n, bits, qweight_out), "pack");
  return GPTQ_OK;
}

gptq_status gptq_dequant_matmul(void* stream, const void* X, int32_t xdt, int64_t M, int64_t n, int64_t ldx,
                                const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                                const int32_t* perm, int64_t d_out, int32_t bits, int32_t group, float* Y,
                                int64_t ldy, void* workspace, size_t ws_bytes) {
  gptq_status st = dq_check(M, n, d_out, bits, group);
  if (st != GPTQ_OK) return st;
  if (xdt != GPTQ_BF16) return fail(GPTQ_EINVAL, "dequant_matmul takes bf16 activations");
  if (M == 0 || d_out == 0) return GPTQ_OK;
  if (ldy < d_out) return fail(GPTQ_EINVAL, "ldy < d_out");
  if (!Y) return fail(GPTQ_EINVAL, "NULL pointer");
  if (n > 0) {
    if (!X || !qweight || !scales || !zeros) return fail(GPTQ_EINVAL, "NULL pointer");
    if (perm == nullptr && (ldx < n || ldx % 8 != 0 || ((uintptr_t)X & 15) != 0))
      return fail(GPTQ_EINVAL, "X rows must be 16-byte aligned (ldx % 8 == 0, ldx >= n)");
    if (perm != nullptr && ldx < n) return fail(GPTQ_EINVAL, "ldx < n");
    if (((uintptr_t)qweight & 15) != 0) return fail(GPTQ_EINVAL, "qweight must be 16-byte aligned");
  }
  const DqPlan p = dequant_mm_plan(M, n, d_out, bits, group);
  if (p.mtiles > 65535 || p.splits > 65535 || p.otiles > ((int64_t)1 << 31) - 1)
    return fail(GPTQ_EINVAL, "dequant_matmul: M or d_out too large for one launch");
  const int permuted = perm != nullptr && n > 0;
  const size_t xp = dq_xp_bytes(M, n, permuted);
  const size_t need = xp + (p.part_bytes + 255) / 256 * 256;
  if (need > 0) {
    if (!workspace || ((uintptr_t)workspace & 255) != 0) return fail(GPTQ_EINVAL, "workspace: NULL or unaligned");
    if (ws_bytes < need) return fail(GPTQ_EWORKSPACE, "workspace too small");
  }
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* Xs = static_cast<const uint16_t*>(X);
  int64_t ldxs = ldx;
  if (permuted) {
    uint16_t* Xp = static_cast<uint16_t*>(workspace);
    HIP_TRY(launch_gather_cols(s, Xs, M, ldx, n, perm, Xp), "gather columns");
    Xs = Xp;
    ldxs = n;
  }
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + xp);
  HIP_TRY(launch_dequant_mm(s, p, Xs, M, n, ldxs, qweight, scales, zeros, d_out, bits, group, Y, ldy, part),
          "dequant_matmul");
  return GPTQ_OK;
}

}  // extern "C"

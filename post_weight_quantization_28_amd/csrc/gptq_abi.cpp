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
int g_prof_level = 0;   // 0 off, 1 the coarse classes, 2 also the phases of quantize_layer
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
// when timing is enabled at `level` or above.
class Timed {
 public:
  Timed(int cls, hipStream_t s, int level = 1) : cls_(cls), s_(s) {
    if (g_prof_level < level) return;
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

// Far field in pairs of super-blocks: after the first of a pair only the
// next super-block's columns are updated (a narrow product, the bridge);
// after the second, one product with both super-blocks' errors (K = 2 sw)
// updates everything to the right. The weights right of the pair are then
// read and written once per pair instead of twice, which is what bounds the
// far field of a large layer; on small ones the extra bridge launches cost
// more than that saves.
constexpr int64_t kPairMinWeights = (int64_t)1 << 27;   // d_out * n
bool pair_far_field(int64_t d_out, int64_t n, const gptq_params* p) {
  return use_two_level(n, p) && d_out * n >= kPairMinWeights;
}

// Super-panel width and the narrowest matrix factorised in two levels (see
// factor_panels).
constexpr int64_t kSuper = 2048;
constexpr int64_t kTwoLevelMinN = 6144;

struct QLayout {
  size_t status, lam, diag, perm, invperm, A, X, Wf, E, Ehi, Elo, Uhi, Ulo, codes, loss, Sp, Ip, total;
};

int64_t inv_x6_pieces(int64_t n);

QLayout q_layout(int64_t d_out, int64_t n, const gptq_params* p) {
  QLayout L{};
  Carver c;
  const bool two = d_out > 0 && use_two_level(n, p);
  const int64_t ew = two ? super_width(p) : p->block;
  const int64_t ewh = pair_far_field(d_out, n, p) ? 2 * ew : ew;   // columns of Ehi / Elo
  L.status = c.take(sizeof(DevStatus));
  L.lam = c.take(sizeof(double));
  L.diag = c.take(sizeof(float) * n);
  L.perm = c.take(sizeof(int32_t) * n);
  L.invperm = c.take(sizeof(int32_t) * n);
  L.A = c.take(sizeof(float) * n * n);
  L.X = c.take(sizeof(float) * n * n);
  L.Wf = c.take(sizeof(float) * d_out * n);
  L.E = c.take(sizeof(float) * d_out * ew);
  L.Ehi = c.take(two ? sizeof(uint16_t) * eh_elems(d_out, ewh) : 0);
  L.Elo = c.take(two ? sizeof(uint16_t) * eh_elems(d_out, ewh) : 0);
  L.Uhi = c.take(two ? sizeof(uint16_t) * n * n : 0);
  L.Ulo = c.take(two ? sizeof(uint16_t) * n * n : 0);
  L.codes = c.take((size_t)d_out * p->n_quant);
  L.loss = c.take(sizeof(float) * d_out);
  // the bf16 pieces of a super-panel for the two-level factorisation's product
  L.Sp = c.take(n >= kTwoLevelMinN ? sizeof(uint16_t) * syrk_x6_pieces(n, kSuper) : 0);
  // the bf16 pieces of the inverse's largest six-product block product
  L.Ip = c.take(sizeof(uint16_t) * inv_x6_pieces(n));
  L.total = c.off;
  return L;
}

// The parameter block grows at its end; fields past a caller's struct_size
// take their defaults.
constexpr size_t kParamsMin = offsetof(gptq_params, sym);
int params_sym(const gptq_params* p) {
  return p->struct_size >= offsetof(gptq_params, sym) + sizeof(int32_t) ? p->sym : 0;
}
// scale_fp16 arrived with `reserved`, which grew the block from 40 to 48
// bytes: a 40-byte block predates it (its bytes 36..39 are padding).
int params_scale16(const gptq_params* p) {
  return p->struct_size >= offsetof(gptq_params, reserved) + sizeof(int32_t) ? p->scale_fp16 : 0;
}
static_assert(offsetof(gptq_params, reserved) + sizeof(int32_t) > 40, "the block must grow past 40 bytes");

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
  const int s16 = params_scale16(p);
  if (s16 != 0 && s16 != 1) return fail(GPTQ_EINVAL, "scale_fp16 must be 0 or 1");
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
// Wide matrices are factorised in two levels. The 64-column panels of a
// super-panel of kSuper columns update only the super-panel's own columns;
// when its last panel is solved, one symmetric rank-kSuper product applies
// all of them to the trailing matrix at once. The trailing matrix is then
// read and written n / kSuper times instead of n / 64 times, and that
// traffic is what bounds the K = 64 updates of a wide matrix. Narrower
// matrices keep one level: their late panels are bound by the leaf chain,
// and the per-super-panel product and leaf launch would only add to it.

// Phase 2's block products go to the six-product bf16 kernels (fp32
// accuracy, see syrk.hip) for the pairs of blocks of h >= kInvX6MinH rows
// whose first product has at least 1024 tiles of 128 x 128, i.e. two rounds
// of two workgroups per CU. Smaller ones stay on the fp32 MFMA GEMM: with
// one 128 x 128 workgroup per CU and K ranges up to 2048 a lone tile's
// stage chain is slower than the fp32 kernel's four 64 x 64 tiles per CU
// (measured: factorisation of a 4096-wide matrix 1.76 ms with the fp32
// products, 1.84 with its 2048-row level on the six-product kernels;
// 11008 wide 11.18 -> 10.20 ms and 28672 wide 128.0 -> 108.0 ms with the
// levels of 1024 or more tiles moved to them).
constexpr int64_t kInvX6MinH = 1024;
constexpr int64_t kInvX6MinTiles = 1024;
bool inv_x6(int64_t h, int64_t hj, int64_t batch) {
  return h >= kInvX6MinH && ceil_div(h, 128) * ceil_div(hj, 128) * batch >= kInvX6MinTiles;
}

// Scratch for the pieces of the largest such product (bf16 elements).
int64_t inv_x6_pieces(int64_t n) {
  int64_t need = 0;
  for (int64_t h = kLeaf; h < n; h *= 2) {
    const int64_t full = n / (2 * h);
    const int64_t bp_last = full * 2 * h + h;
    const int64_t hj_last = bp_last < n ? n - bp_last : 0;
    auto take = [&](int64_t hj, int64_t batch) {
      if (batch <= 0 || hj <= 0 || !inv_x6(h, hj, batch)) return;
      need = std::max(need, batch * (x6_op_elems(h, h) + x6_op_elems(hj, h)));
      need = std::max(need, batch * (x6_op_elems(hj, hj) + x6_op_elems(h, hj)));
    };
    take(h, full);
    take(hj_last, 1);
  }
  return need;
}

// Right-looking Cholesky of the flipped matrix A with the inverse X = L^{-1}
// carried along (see factor.hip): two launches per 64-column panel.
hipError_t factor_panels(hipStream_t s, float* A, float* X, int64_t n, const int32_t* perm,
                         DevStatus* st, uint16_t* pieces,
                         uint16_t* ipieces) {
  hipError_t e;
  const int64_t S = n >= kTwoLevelMinN ? kSuper : n;
  // ---- phase 1: Cholesky, leaves write D = L11^{-1} into X's diagonal
  if ((e = launch_leaf(s, A, X, n, 0, std::min<int64_t>(kLeaf, n), perm, st)) != hipSuccess) return e;
  for (int64_t s0 = 0; s0 < n; s0 += S) {
    const int64_t s1 = std::min<int64_t>(s0 + S, n);
    for (int64_t k0 = s0; k0 < s1; k0 += kLeaf) {
      const int64_t m = std::min<int64_t>(kLeaf, n - k0);
      const int64_t k1 = k0 + m, r = n - k1;
      if (r == 0) break;
      const float* D = X + k0 * n + k0;    // L11^{-1}, lower
      float* L21 = A + k1 * n + k0;
      // L21 = A21 D^T in place (m == 64 whenever rows remain below the panel)
      if ((e = launch_panel_solve(s, L21, D, n, r)) != hipSuccess) return e;
      if (k1 == s1) break;                 // the super-panel's last panel: the product below updates
      // One launch: the next diagonal block (m2 rows) is updated and factored
      // by its own workgroup while the rest runs
      //   A[k1+m2:, k1:s1] -= L21[m2:] L21[:s1-k1]^T   (lower, i.e. j <= i + m2)
      const int64_t m2 = std::min<int64_t>(kLeaf, r);
      SlabArgs g3{};
      g3.M = r - m2; g3.N = s1 - k1; g3.K = m;
      g3.A = L21 + m2 * n; g3.lda = n;
      g3.B = L21; g3.ldb = n; g3.tb = 1;
      g3.C = A + (k1 + m2) * n + k1; g3.ldc = n;
      g3.alpha = -1.f; g3.beta = 1.f;
      g3.lower_only = 1; g3.lower_off = m2;
      LeafTask lt{L21, A, X, n, k1, (int)m2, (int)m, perm, st};
      if ((e = launch_slab_leaf(s, g3, lt)) != hipSuccess) return e;
    }
    if (s1 < n) {
      // A[s1:, s1:] -= L[s1:, s0:s1] L[s1:, s0:s1]^T on the lower tiles,
      // then the next super-panel's first leaf
      GemmArgs g{};
      g.M = n - s1; g.N = n - s1; g.K = s1 - s0;
      g.A = A + s1 * n + s0; g.lda = n; g.ta = 0;
      g.B = A + s1 * n + s0; g.ldb = n; g.tb = 1;
      g.C = A + s1 * n + s1; g.ldc = n;
      g.alpha = -1.f; g.beta = 1.f; g.batch = 1;
      if (pieces && syrk_x6_ok(g.N, g.K, g.lda, g.A, g.ldc, g.C))
        e = launch_syrk_x6(s, g.A, g.lda, g.C, g.ldc, g.N, g.K, pieces);
      else
        e = launch_syrk_f32(s, g);
      if (e != hipSuccess) return e;
      if ((e = launch_leaf(s, A, X, n, s1, std::min<int64_t>(kLeaf, n - s1), perm, st)) != hipSuccess) return e;
    }
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
    const bool x6f = ipieces && full > 0 && inv_x6(h, h, full);
    const bool x6p = ipieces && hj_last > 0 && inv_x6(h, hj_last, 1);
    if (x6f || x6p) {
      // the same two products per pair, each operand split into its pieces
      // first: g1's A is X_ii read down its columns (X_ii^T), its B the rows
      // of L_ji; g2's A the rows of X_jj, its B the rows of T^T
      auto x6 = [&](const GemmArgs& g1, const GemmArgs& g2) -> hipError_t {
        const int bt = std::max(g1.batch, 1);
        hipError_t r;
        if ((r = x6_split(s, g1.M, g1.N, g1.K, bt, X6Operand{g1.A, g1.lda, g1.sA, 1},
                          X6Operand{g1.B, g1.ldb, g1.sB, 0}, ipieces)) != hipSuccess)
          return r;
        {
          Timed t(GPTQ_PROF_INVERSE_X6, s, 2);
          if ((r = x6_product(s, g1.M, g1.N, g1.K, bt, g1.C, g1.ldc, g1.sC, g1.alpha, g1.kmode, ipieces)) !=
              hipSuccess)
            return r;
        }
        if ((r = x6_split(s, g2.M, g2.N, g2.K, bt, X6Operand{g2.A, g2.lda, g2.sA, 0},
                          X6Operand{g2.B, g2.ldb, g2.sB, 0}, ipieces)) != hipSuccess)
          return r;
        Timed t(GPTQ_PROF_INVERSE_X6, s, 2);
        return x6_product(s, g2.M, g2.N, g2.K, bt, g2.C, g2.ldc, g2.sC, g2.alpha, g2.kmode, ipieces);
      };
      auto f32 = [&](const GemmArgs& g1, const GemmArgs& g2) -> hipError_t {
        hipError_t r;
        if ((r = launch_gemm_pair(s, g1, nullptr)) != hipSuccess) return r;
        return launch_gemm_pair(s, g2, nullptr);
      };
      if (full > 0 && (e = x6f ? x6(f1, f2) : f32(f1, f2)) != hipSuccess) return e;
      if (hj_last > 0 && (e = x6p ? x6(p1, p2) : f32(p1, p2)) != hipSuccess) return e;
      continue;
    }
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
  uint16_t* pieces = L.Sp != L.total && n >= kTwoLevelMinN ? reinterpret_cast<uint16_t*>(ws + L.Sp) : nullptr;
  uint16_t* ipieces = inv_x6_pieces(n) > 0 ? reinterpret_cast<uint16_t*>(ws + L.Ip) : nullptr;
  HIP_TRY(factor_panels(s, A, X, n, perm, st, pieces, ipieces), "factor");
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

// ---------------------------------------------------------------- EoRA
// Top-r eigenpairs of G = D H D^T (D = W - W_hat) by block subspace
// iteration: Y = G Q, Q = orth(Y) by CholeskyQR on unit columns (Y's
// columns scaled to length 1, C = Y^T Y with a unit diagonal, U with
// U^T U = (C + lambda I)^{-1} from this library's factorisation, Q = Y U^T;
// lambda = 1e-5 keeps a nearly rank-deficient block factorable in fp32),
// then Rayleigh-Ritz: S = Q^T G Q, S = V Theta V^T (Jacobi), U_r = Q V_r.
constexpr int kEoraMaxRank = 64;
constexpr int kEoraOversample = 64;
constexpr int kEoraDefaultIters = 24;

int eora_block(int64_t d_out, int rank) {
  int64_t k = std::min<int64_t>(rank + kEoraOversample, 128);
  if (k > d_out) k = d_out;
  if (k & 1) k += 1;            // Jacobi pairs indices: k even (at most one direction past d_out)
  return (int)k;
}

struct ELayout {
  size_t status, D, T, G, Y, Q, C, S, V, theta, fac, part, total;
  QLayout fl;
  int k;
};

// Split-K for the skinny products of the subspace iteration (few output
// tiles, long K): the K range is cut into equal chunks run as one batched
// launch into fp32 partials (and one launch for a ragged rest), then summed
// in a fixed order. At most kSplitMax + 1 partials.
constexpr int kSplitMax = 64;

int split_count(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ceil_div(M, 64) * ceil_div(N, 64);
  if (tiles >= 512 || K < 256) return 1;
  int64_t sp = std::min<int64_t>(ceil_div(512, tiles), K / 128);
  return (int)std::max<int64_t>(1, std::min<int64_t>(sp, kSplitMax));
}

// C (M x N, contiguous) = op(A) op(B) with split K. ta/tb as GemmArgs.
hipError_t gemm_splitk(hipStream_t s, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int ta,
                       const float* B, int64_t ldb, int tb, float* C, float* part) {
  const int sp = split_count(M, N, K);
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.ta = ta;
  g.B = B; g.ldb = ldb; g.tb = tb;
  g.C = C; g.ldc = N;
  g.alpha = 1.f; g.beta = 0.f; g.batch = 1;
  if (sp == 1) return launch_gemm_f32(s, g);
  const int64_t kc = K / sp, rest = K - kc * sp;
  g.K = kc; g.batch = sp;
  g.sA = ta ? kc * lda : kc;         // the chunk's first k: row of a K x M store, column of an M x K one
  g.sB = tb ? kc : kc * ldb;
  g.C = part; g.sC = M * N;
  hipError_t e = launch_gemm_f32(s, g);
  if (e != hipSuccess) return e;
  int np = sp;
  if (rest > 0) {
    GemmArgs r = g;
    r.K = rest; r.batch = 1;
    r.A = A + (ta ? sp * kc * lda : sp * kc);
    r.B = B + (tb ? sp * kc : sp * kc * ldb);
    r.C = part + (int64_t)sp * M * N;
    if ((e = launch_gemm_f32(s, r)) != hipSuccess) return e;
    ++np;
  }
  return launch_sum_partials(s, part, np, M * N, C);
}

gptq_params eora_factor_params(int k) {
  gptq_params fp{};
  fp.struct_size = sizeof(gptq_params);
  fp.bits = 4; fp.group = 8; fp.block = 32;
  fp.damp = 1e-5f; fp.act_order = 0; fp.n_quant = k; fp.sym = 0;
  return fp;
}

ELayout e_layout(int64_t d_out, int64_t n, int rank, int with_h) {
  ELayout L{};
  Carver c;
  L.k = eora_block(d_out, rank);
  const int64_t k = L.k;
  const gptq_params fp = eora_factor_params(L.k);
  L.fl = q_layout(0, k, &fp);
  L.status = c.take(sizeof(DevStatus));
  L.D = c.take(sizeof(float) * d_out * n);
  L.T = c.take(with_h ? sizeof(float) * d_out * n : 0);
  L.G = c.take(sizeof(float) * d_out * d_out);
  L.Y = c.take(sizeof(float) * d_out * k);
  L.Q = c.take(sizeof(float) * d_out * k);
  L.C = c.take(sizeof(float) * k * k);
  L.S = c.take(sizeof(float) * k * k);
  L.V = c.take(sizeof(float) * k * k);
  L.theta = c.take(sizeof(float) * k);
  L.fac = c.take(L.fl.total);
  // split-K partials of the three skinny products (G Q, the k x k Gram and
  // Rayleigh matrices, A = U_r^T D): (splits + 1) x M x N floats each
  int64_t mx = 0;
  const int64_t uses[3][3] = {{d_out, k, d_out}, {k, k, d_out}, {rank, n, d_out}};
  for (const auto& u : uses) {
    const int sp = split_count(u[0], u[1], u[2]);
    if (sp > 1) mx = std::max<int64_t>(mx, (sp + 1) * u[0] * u[1]);
  }
  L.part = c.take(sizeof(float) * mx);
  L.total = c.off;
  return L;
}

GemmArgs gemm(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, int ta, const float* B, int64_t ldb,
              int tb, float* C, int64_t ldc) {
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.ta = ta;
  g.B = B; g.ldb = ldb; g.tb = tb;
  g.C = C; g.ldc = ldc;
  g.alpha = 1.f; g.beta = 0.f; g.batch = 1;
  return g;
}

// Q = Y U^T with U^T U = (Y^T Y + lambda I)^{-1} after Y's columns are
// scaled to unit length (in place): columns of Q orthonormal (up to
// lambda) and spanning Y's columns.
gptq_status eora_orth(hipStream_t s, float* Y, float* Q, int64_t d, const ELayout& L, char* ws) {
  const int64_t k = L.k;
  float* C = reinterpret_cast<float*>(ws + L.C);
  HIP_TRY(launch_col_normalize(s, Y, d, (int)k), "eora normalize");
  HIP_TRY(gemm_splitk(s, k, k, d, Y, k, 1, Y, k, 0, C, reinterpret_cast<float*>(ws + L.part)), "eora gram");
  const gptq_params fp = eora_factor_params(L.k);
  gptq_status st = enqueue_factor(s, C, k, &fp, ws + L.fac, L.fl);
  if (st != GPTQ_OK) return st;
  const float* U = reinterpret_cast<const float*>(ws + L.fac + L.fl.A);
  HIP_TRY(launch_gemm_f32(s, gemm(d, k, k, Y, k, 0, U, k, 1, Q, k)), "eora orth");
  return GPTQ_OK;
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
  g_prof_level = enable <= 0 ? 0 : (enable == 1 ? 1 : 2);
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
  {
    Timed ph(GPTQ_PROF_FACTOR, s, 2);
    if ((st = enqueue_factor(s, H, n, p, ws, L, two ? Uhi : nullptr, two ? Ulo : nullptr)) != GPTQ_OK) return st;
  }
  {
    Timed ph(GPTQ_PROF_PREP_FINISH, s, 2);
    HIP_TRY(launch_w_prep(s, W, wdt == GPTQ_BF16, d_out, n, ldw, p->act_order ? perm : nullptr, Wf, dst),
            "w prep");
    HIP_TRY(launch_fill_f32(s, loss, (size_t)d_out, 0.f), "fill");
  }
  // Two-level lazy batch. Inside a super-block [s0, s1) each block updates
  // the super-block's later columns at once (fp32, K = B); when the
  // super-block is done, all of its errors update the columns right of it
  // in one split-bf16 product (K = s1 - s0). Without the split path the
  // super-block is the block itself and the far field is fp32. With B = 128,
  // whole blocks and groups inside a block, the in-super-block update is
  // taken left-looking by the sweep kernel itself (each block first applies
  // the errors of the super-block's earlier blocks to its own columns).
  const bool fused = two && B == 128 && p->group <= B && nq % B == 0 && sw == 512;
  // the fused path takes a whole super-block per launch when U's rows are
  // 16-byte aligned (the tile loads are unpredicated float4)
  const bool sbl = fused && n % 4 == 0 && ((uintptr_t)U & 15) == 0;
  // far field in pairs of super-blocks (see pair_far_field): the second of a
  // pair writes its bf16 error parts sw columns to the right of the first's
  const bool pair = two && pair_far_field(d_out, n, p);
  const int64_t ldeh = pair ? 2 * sw : sw;
  bool owed = false;     // a first-of-pair super-block whose far field right of the next one is pending
  int64_t ps0 = 0;       // its first column
  for (int64_t s0 = 0; s0 < nq; s0 += sw) {
    const int64_t s1 = std::min<int64_t>(s0 + sw, nq);
    const int64_t eoff = pair && owed ? sw : 0;   // this super-block's columns in Ehi / Elo
    if (sbl) {
      SweepArgs a{};
      a.Wf = Wf; a.ldw = n; a.U = U; a.ldu = n; a.d_out = d_out; a.i0 = s0; a.ncols = s1 - s0;
      a.block = B; a.group = p->group; a.bits = p->bits; a.sym = params_sym(p); a.scale16 = params_scale16(p);
      a.gbase = s0 / p->group;
      a.gshift = 31;
      if (p->group < B)
        for (int sh = 0; sh < 31; ++sh)
          if ((1 << sh) == p->group) a.gshift = sh;
      a.scales = out->scales; a.zeros = out->zeros; a.ngroups = nq / p->group;
      a.codes = codes; a.n_quant = nq; a.E = E; a.lde = sw; a.row_loss = loss; a.st = dst;
      a.Esb = E; a.kb = 0;
      a.Ehi = s1 < n ? Ehi : nullptr;
      a.Elo = s1 < n ? Elo : nullptr;
      a.ldeh = ldeh;
      a.ehcol = eoff;
      Timed ph(GPTQ_PROF_SWEEP, s, 2);
      HIP_TRY(launch_sweep_super(s, a), "sweep");
    }
    for (int64_t i0 = s0; i0 < s1 && !sbl; i0 += B) {
      const int64_t nc = std::min<int64_t>(B, s1 - i0);
      float* Eb = E + (i0 - s0);
      SweepArgs a{};
      a.Wf = Wf; a.ldw = n; a.U = U; a.ldu = n; a.d_out = d_out; a.i0 = i0; a.ncols = nc;
      a.block = B; a.group = p->group; a.bits = p->bits; a.sym = params_sym(p); a.scale16 = params_scale16(p);
      a.gbase = i0 / p->group;
      a.gshift = 31;
      if (p->group < B)
        for (int sh = 0; sh < 31; ++sh)
          if ((1 << sh) == p->group) a.gshift = sh;
      a.scales = out->scales; a.zeros = out->zeros; a.ngroups = nq / p->group;
      a.codes = codes; a.n_quant = nq; a.E = Eb; a.lde = sw; a.row_loss = loss; a.st = dst;
      a.Esb = E; a.kb = fused ? i0 - s0 : 0;
      a.Ehi = two && s1 < n ? Ehi : nullptr;
      a.Elo = two && s1 < n ? Elo : nullptr;
      a.ldeh = ldeh;
      a.ehcol = eoff + (i0 - s0);
      Timed ph(GPTQ_PROF_SWEEP, s, 2);
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
      // rows [k0, s1) of U and columns [s1, s1 + N) of W: the first of a
      // pair updates only the next super-block (the bridge), the second
      // applies both super-blocks' errors to everything to its right
      const bool bridge = pair && !owed && s1 < nq;
      const int64_t k0 = pair && owed ? ps0 : s0;
      TrailArgs t{};
      t.M = d_out; t.N = bridge ? std::min<int64_t>(s1 + sw, nq) - s1 : n - s1; t.K = s1 - k0;
      t.Ahi = Ehi; t.Alo = Elo; t.lda = ldeh;
      t.Bhi = Uhi + k0 * n + s1; t.Blo = Ulo + k0 * n + s1; t.ldb = n;
      t.C = Wf + s1; t.ldc = n;
      Timed ph(GPTQ_PROF_FARFIELD, s, 2);
      HIP_TRY(launch_trail_x3(s, t), "far-field update");
      owed = bridge;
      if (bridge) ps0 = s0;
    }
  }
  Timed ph(GPTQ_PROF_PREP_FINISH, s, 2);
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

}  // extern "C"

namespace {

// Bytes of scratch one gptq_dequant_matmul call needs (the gathered
// activations when permuted, then the fp32 partials); valid arguments only.
size_t dq_need(int64_t M, int64_t n, int64_t d_out, int32_t bits, int32_t group, int permuted) {
  const DqPlan p = dequant_mm_plan(M, n, d_out, bits, group);
  return dq_xp_bytes(M, n, permuted) + (p.part_bytes + 255) / 256 * 256;
}

// Argument checks shared by both dequant_matmul entry points (host only,
// nothing enqueued). *run = 0 when there is nothing to launch.
gptq_status dq_validate(const void* X, int32_t xdt, int64_t M, int64_t n, int64_t ldx, const uint32_t* qweight,
                        const float* scales, const uint8_t* zeros, const int32_t* perm, int64_t d_out,
                        int32_t bits, int32_t group, float* Y, int64_t ldy, int* run) {
  *run = 0;
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
  *run = 1;
  return GPTQ_OK;
}

// The launches of one product, with `scratch` (at least dq_need bytes,
// 256-byte aligned) already checked by the caller.
gptq_status dq_enqueue(hipStream_t s, const void* X, int64_t M, int64_t n, int64_t ldx, const uint32_t* qweight,
                       const float* scales, const uint8_t* zeros, const int32_t* perm, int64_t d_out,
                       int32_t bits, int32_t group, float* Y, int64_t ldy, void* scratch) {
  const DqPlan p = dequant_mm_plan(M, n, d_out, bits, group);
  const int permuted = perm != nullptr && n > 0;
  const size_t xp = dq_xp_bytes(M, n, permuted);
  const uint16_t* Xs = static_cast<const uint16_t*>(X);
  int64_t ldxs = ldx;
  if (permuted) {
    uint16_t* Xp = static_cast<uint16_t*>(scratch);
    HIP_TRY(launch_gather_cols(s, Xs, M, ldx, n, perm, Xp), "gather columns");
    Xs = Xp;
    ldxs = n;
  }
  float* part = reinterpret_cast<float*>(static_cast<char*>(scratch) + xp);
  HIP_TRY(launch_dequant_mm(s, p, Xs, M, n, ldxs, qweight, scales, zeros, d_out, bits, group, Y, ldy, part),
          "dequant_matmul");
  return GPTQ_OK;
}

// ---- the allocation-free variant's scratch: one array per GPU, in the code
// object's device memory (each device that loads the library holds its own
// copy until the process ends). Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[GPTQ_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // indexed by device ordinal; nullptr = not looked up yet

gptq_status scratch_for_current_device(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255) != 0) return fail(GPTQ_EHIP, "static scratch address is NULL or unaligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GPTQ_OK;
}

}  // namespace

extern "C" {

gptq_status gptq_dequant_matmul(void* stream, const void* X, int32_t xdt, int64_t M, int64_t n, int64_t ldx,
                                const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                                const int32_t* perm, int64_t d_out, int32_t bits, int32_t group, float* Y,
                                int64_t ldy, void* workspace, size_t ws_bytes) {
  int run = 0;
  gptq_status st = dq_validate(X, xdt, M, n, ldx, qweight, scales, zeros, perm, d_out, bits, group, Y, ldy, &run);
  if (st != GPTQ_OK || !run) return st;
  const size_t need = dq_need(M, n, d_out, bits, group, perm != nullptr && n > 0);
  if (need > 0) {
    if (!workspace || ((uintptr_t)workspace & 255) != 0) return fail(GPTQ_EINVAL, "workspace: NULL or unaligned");
    if (ws_bytes < need) return fail(GPTQ_EWORKSPACE, "workspace too small");
  }
  return dq_enqueue((hipStream_t)stream, X, M, n, ldx, qweight, scales, zeros, perm, d_out, bits, group, Y, ldy,
                    workspace);
}

gptq_status gptq_dequant_matmul_noalloc(void* stream, const void* X, int32_t xdt, int64_t M, int64_t n,
                                        int64_t ldx, const uint32_t* qweight, const float* scales,
                                        const uint8_t* zeros, const int32_t* perm, int64_t d_out, int32_t bits,
                                        int32_t group, float* Y, int64_t ldy) {
  int run = 0;
  gptq_status st = dq_validate(X, xdt, M, n, ldx, qweight, scales, zeros, perm, d_out, bits, group, Y, ldy, &run);
  if (st != GPTQ_OK || !run) return st;
  const size_t need = dq_need(M, n, d_out, bits, group, perm != nullptr && n > 0);
  if (need > (size_t)GPTQ_NOALLOC_SCRATCH_BYTES) {
    char msg[160];
    snprintf(msg, sizeof msg, "dequant_matmul_noalloc: this product needs %zu bytes of scratch; the static "
             "scratch holds %zu (use gptq_dequant_matmul with a workspace)", need,
             (size_t)GPTQ_NOALLOC_SCRATCH_BYTES);
    return fail(GPTQ_EINVAL, msg);
  }
  void* ws = nullptr;
  if (need > 0 && (st = scratch_for_current_device(&ws)) != GPTQ_OK) return st;
  return dq_enqueue((hipStream_t)stream, X, M, n, ldx, qweight, scales, zeros, perm, d_out, bits, group, Y, ldy,
                    ws);
}


// ---------------------------------------------------------------- EoRA
gptq_status gptq_eora_workspace_bytes(int64_t d_out, int64_t n, int32_t rank, int32_t with_h, size_t* bytes) {
  if (!bytes) return fail(GPTQ_EINVAL, "bytes is NULL");
  if (d_out < 1 || n < 1 || d_out > ((int64_t)1 << 30) || n > ((int64_t)1 << 30))
    return fail(GPTQ_EINVAL, "need 1 <= d_out, n <= 2^30");
  if (rank < 1 || rank > kEoraMaxRank || rank > d_out) return fail(GPTQ_EINVAL, "rank must be in [1, min(64, d_out)]");
  *bytes = e_layout(d_out, n, rank, with_h != 0).total;
  return GPTQ_OK;
}

gptq_status gptq_eora(void* stream, const void* W, gptq_dtype wdt, const float* W_hat, int64_t d_out, int64_t n,
                      int64_t ldw, const float* H, int32_t rank, int32_t iters, float* B, float* A, float* sigma,
                      void* workspace, size_t workspace_bytes) {
  size_t need = 0;
  gptq_status st = gptq_eora_workspace_bytes(d_out, n, rank, H != nullptr, &need);
  if (st != GPTQ_OK) return st;
  if (wdt != GPTQ_BF16 && wdt != GPTQ_F32) return fail(GPTQ_EINVAL, "bad dtype");
  if (!W || !W_hat || !B || !A || !sigma) return fail(GPTQ_EINVAL, "NULL pointer");
  if (ldw < n) return fail(GPTQ_EINVAL, "ldw < n");
  if (iters < 0 || iters > 1000) return fail(GPTQ_EINVAL, "iters must be in [0, 1000]");
  if ((st = check_ws(workspace, workspace_bytes, need)) != GPTQ_OK) return st;
  const int it_n = iters == 0 ? kEoraDefaultIters : iters;
  hipStream_t s = (hipStream_t)stream;
  char* ws = reinterpret_cast<char*>(workspace);
  const ELayout L = e_layout(d_out, n, rank, H != nullptr);
  const int64_t k = L.k, d = d_out;
  DevStatus* dst = reinterpret_cast<DevStatus*>(ws + L.status);
  float* D = reinterpret_cast<float*>(ws + L.D);
  float* T = reinterpret_cast<float*>(ws + L.T);
  float* G = reinterpret_cast<float*>(ws + L.G);
  float* Y = reinterpret_cast<float*>(ws + L.Y);
  float* Q = reinterpret_cast<float*>(ws + L.Q);
  float* S = reinterpret_cast<float*>(ws + L.S);
  float* V = reinterpret_cast<float*>(ws + L.V);
  float* theta = reinterpret_cast<float*>(ws + L.theta);
  HIP_TRY(launch_status_init(s, dst), "status init");
  HIP_TRY(launch_eora_delta(s, W, wdt == GPTQ_BF16, ldw, W_hat, d, n, D, dst), "eora delta");
  // G = D H D^T (plain SVD of D when H is NULL: G = D D^T)
  if (H) {
    HIP_TRY(launch_gemm_f32(s, gemm(d, n, n, D, n, 0, H, n, 0, T, n)), "eora D H");
    HIP_TRY(launch_gemm_f32(s, gemm(d, d, n, T, n, 0, D, n, 1, G, d)), "eora G");
  } else {
    HIP_TRY(launch_gemm_f32(s, gemm(d, d, n, D, n, 0, D, n, 1, G, d)), "eora G");
  }
  // start block and subspace iteration
  HIP_TRY(launch_eora_start(s, Q, d, (int)k), "eora start");
  float* part = reinterpret_cast<float*>(ws + L.part);
  HIP_TRY(gemm_splitk(s, d, k, d, G, d, 0, Q, k, 0, Y, part), "eora G Q");
  for (int it = 0; it < it_n; ++it) {
    if ((st = eora_orth(s, Y, Q, d, L, ws)) != GPTQ_OK) return st;
    HIP_TRY(gemm_splitk(s, d, k, d, G, d, 0, Q, k, 0, Y, part), "eora G Q");
  }
  // CholeskyQR2 for the final basis, then Rayleigh-Ritz
  if ((st = eora_orth(s, Y, Q, d, L, ws)) != GPTQ_OK) return st;
  if ((st = eora_orth(s, Q, Y, d, L, ws)) != GPTQ_OK) return st;       // Y holds the basis now
  HIP_TRY(gemm_splitk(s, d, k, d, G, d, 0, Y, k, 0, Q, part), "eora G Q");
  HIP_TRY(gemm_splitk(s, k, k, d, Y, k, 1, Q, k, 0, S, part), "eora Rayleigh quotient");
  HIP_TRY(launch_sym_eig_jacobi(s, S, (int)k, theta, V), "eora Jacobi");
  // U_r = basis V[:, :r] into B, A = U_r^T D, then the singular-value scaling
  HIP_TRY(launch_gemm_f32(s, gemm(d, rank, k, Y, k, 0, V, k, 0, B, rank)), "eora U_r");
  HIP_TRY(gemm_splitk(s, rank, n, d, B, rank, 1, D, n, 0, A, part), "eora A");
  HIP_TRY(launch_eora_finish(s, theta, rank, sigma, B, d, rank, A, n), "eora finish");
  // device status: the difference, then the last factorisation (NaN in H
  // reaches the Gram matrix it factors)
  int64_t col = -1;
  if ((st = read_status(s, dst, nullptr, &col)) != GPTQ_OK) return st;
  return read_status(s, reinterpret_cast<DevStatus*>(ws + L.fac + L.fl.status), nullptr, nullptr);
}

// ---------------------------------------------------------------- OLrC / Bid-Up refinement
namespace {
struct RLayout {
  size_t Qh, T, D, G, Delta, B0, A0, sig, eora, total;
};

RLayout r_layout(int64_t d_out, int64_t n, int rank) {
  RLayout L{};
  Carver c;
  L.Qh = c.take(sizeof(float) * d_out * n);
  L.T = c.take(sizeof(float) * d_out * n);
  L.D = c.take(sizeof(float) * d_out * n);
  L.G = c.take(sizeof(float) * d_out * n);
  L.Delta = c.take(sizeof(float) * d_out * 128);
  L.sig = c.take(sizeof(float) * 64);
  L.eora = c.take(e_layout(d_out, n, rank, 1).total);
  L.total = c.off;
  return L;
}
}  // namespace

gptq_status gptq_refine_workspace_bytes(int64_t d_out, int64_t n, int32_t rank, size_t* bytes) {
  size_t e = 0;
  gptq_status st = gptq_eora_workspace_bytes(d_out, n, rank, 1, &e);
  if (st != GPTQ_OK) return st;
  *bytes = r_layout(d_out, n, rank).total;
  return GPTQ_OK;
}

gptq_status gptq_refine_lowrank(void* stream, const void* W, gptq_dtype wdt, int64_t d_out, int64_t n, int64_t ldw,
                                const float* H, int32_t bits, int32_t group, const int32_t* g_idx,
                                const float* scales, const uint8_t* zeros, uint8_t* codes, int32_t rank,
                                int32_t cycles, int32_t passes, float* B, float* A, float* w_hat,
                                void* workspace, size_t workspace_bytes) {
  size_t need = 0;
  gptq_status st = gptq_refine_workspace_bytes(d_out, n, rank, &need);
  if (st != GPTQ_OK) return st;
  if (wdt != GPTQ_BF16 && wdt != GPTQ_F32) return fail(GPTQ_EINVAL, "bad dtype");
  if (bits < 2 || bits > 8) return fail(GPTQ_EINVAL, "bits must be in [2, 8]");
  if (group < 1 || n % group != 0) return fail(GPTQ_EINVAL, "group must divide n");
  if (cycles < 1 || cycles > 100 || passes < 1 || passes > 100) return fail(GPTQ_EINVAL, "cycles and passes in [1, 100]");
  if (!W || !H || !g_idx || !scales || !zeros || !codes || !B || !A) return fail(GPTQ_EINVAL, "NULL pointer");
  if (ldw < n) return fail(GPTQ_EINVAL, "ldw < n");
  if ((st = check_ws(workspace, workspace_bytes, need)) != GPTQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = reinterpret_cast<char*>(workspace);
  const RLayout L = r_layout(d_out, n, rank);
  const int64_t ng = n / group;
  float* Qh = reinterpret_cast<float*>(ws + L.Qh);
  float* T = reinterpret_cast<float*>(ws + L.T);
  float* D = reinterpret_cast<float*>(ws + L.D);
  float* G = reinterpret_cast<float*>(ws + L.G);
  float* Delta = reinterpret_cast<float*>(ws + L.Delta);
  float* sig = reinterpret_cast<float*>(ws + L.sig);
  void* ews = ws + L.eora;
  const size_t ebytes = e_layout(d_out, n, rank, 1).total;
  HIP_TRY(launch_bid_residual(s, nullptr, codes, scales, zeros, g_idx, ng, d_out, n, Qh), "dequantise");
  for (int cy = 0; cy < cycles; ++cy) {
    // OLrC: the optimal rank-r B A for the current codes (the EoRA problem on W - W_hat)
    if ((st = gptq_eora(stream, W, wdt, Qh, d_out, n, ldw, H, rank, 0, B, A, sig, ews, ebytes)) != GPTQ_OK)
      return st;
    // target T = W - B A
    HIP_TRY(launch_gemm_f32(s, gemm(d_out, n, rank, B, rank, 0, A, n, 0, D, n)), "B A");
    DevStatus* dst = reinterpret_cast<DevStatus*>(ws + L.eora + e_layout(d_out, n, rank, 1).status);
    HIP_TRY(launch_status_init(s, dst), "status init");
    HIP_TRY(launch_eora_delta(s, W, wdt == GPTQ_BF16, ldw, D, d_out, n, T, dst), "target");
    // Bid-Up passes: G = (T - W_hat) H, then blocks of 128 columns with lazy trailing updates
    for (int ps = 0; ps < passes; ++ps) {
      HIP_TRY(launch_bid_residual(s, T, codes, scales, zeros, g_idx, ng, d_out, n, D), "residual");
      HIP_TRY(launch_gemm_f32(s, gemm(d_out, n, n, D, n, 0, H, n, 0, G, n)), "gradient");
      for (int64_t j0 = 0; j0 < n; j0 += 128) {
        const int nb = (int)std::min<int64_t>(128, n - j0);
        HIP_TRY(launch_bidup_block(s, G, n, H, codes, scales, g_idx, ng, d_out, j0, nb, bits, Delta),
                "bid-up block");
        const int64_t j1 = j0 + nb;
        if (j1 < n) {
          GemmArgs g = gemm(d_out, n - j1, nb, Delta, 128, 0, H + j0 * n + j1, n, 0, G + j1, n);
          g.alpha = -1.f;
          g.beta = 1.f;
          HIP_TRY(launch_gemm_f32(s, g), "bid-up trailing update");
        }
      }
    }
    HIP_TRY(launch_bid_residual(s, nullptr, codes, scales, zeros, g_idx, ng, d_out, n, Qh), "dequantise");
    int64_t col = -1;
    if ((st = read_status(s, dst, nullptr, &col)) != GPTQ_OK) return st;
  }
  if (w_hat) HIP_TRY(hipMemcpyAsync(w_hat, Qh, sizeof(float) * d_out * n, hipMemcpyDeviceToDevice, s), "copy w_hat");
  HIP_TRY(hipStreamSynchronize(s), "synchronize");
  return GPTQ_OK;
}

// ---------------------------------------------------------------- round-to-nearest
gptq_status gptq_quantize_rtn(void* stream, const float* X, int64_t rows, int64_t cols, int64_t ldx, int32_t bits,
                              int32_t group, uint8_t* codes, float* scales, uint8_t* zeros, float* x_hat) {
  if (bits < 2 || bits > 8) return fail(GPTQ_EINVAL, "bits must be in [2, 8]");
  if (rows < 0 || cols < 0 || group < 1) return fail(GPTQ_EINVAL, "bad size");
  if (cols % group != 0) return fail(GPTQ_EINVAL, "group must divide cols");
  if (ldx < cols) return fail(GPTQ_EINVAL, "ldx < cols");
  if (cols / group > 2147483647 || rows > 65535) return fail(GPTQ_EINVAL, "too many groups or rows for one launch");
  if (rows * cols == 0) return GPTQ_OK;
  if (!X || !codes || !scales || !zeros) return fail(GPTQ_EINVAL, "NULL pointer");
  HIP_TRY(launch_rtn((hipStream_t)stream, X, ldx, rows, cols, bits, group, codes, scales, zeros, x_hat), "rtn");
  return GPTQ_OK;
}
}  // extern "C"

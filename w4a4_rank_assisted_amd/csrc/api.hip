// api.hip -- the C ABI of libhsq (declared in include/hsq.h): argument
// validation, workspace planning and kernel launches.  No allocation, no
// state, no exceptions across the interface.
#include "hsq.h"
#include "hsq_internal.h"

#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstdint>
#include <mutex>

namespace hsq {

WsLayout plan_workspace(int M, int K, int N, int r, int batch, int group) {
  WsLayout L;
  L.MT = ceil_div(M, kTile);
  L.group = group;
  L.bpg = group / kGroup;
  L.G = K / group;
  L.Gp = padded_groups(K);
  L.SG = scale_groups_stored(K, group);
  L.Mpad = L.MT * kTile;
  // Quantization pass: K is split into slices whose U partials are summed
  // by the contraction kernels.
  L.u_slices = quant_slices(M, K, r, batch, group);
  size_t off = 0;
  L.qa_off = off;
  off = align_up(off + (size_t)L.MT * L.Gp * 1024, 256);
  L.sxs_off = off;
  off = align_up(off + (size_t)L.MT * L.SG * 16 * sizeof(uint16_t), 256);
  L.uw_off = off;
  off = align_up(off + (size_t)L.u_slices * batch * r * L.Mpad * sizeof(float), 256);
  L.part_off = off;
  off = align_up(off + tiled_partial_bytes(M, N, K, r, batch, group), 256);
  L.swr = sw_pair_rows(K, group);
  L.npad = ceil_div(N, kTile) * kTile;
  L.swp_off = off;
  off = align_up(off + (size_t)batch * L.swr * L.npad * 8, 256);
  L.total = off;
  return L;
}

}  // namespace hsq

using namespace hsq;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_sizes(int M, int K, int N, int r, int batch) {
  if (M < 1 || N < 1 || K < 1 || r < 0 || r > kMaxRank || batch < 1 || batch > kMaxBatch)
    return HSQ_E_INVAL;
  if (K % kGroup != 0) return HSQ_E_SHAPE;
  if ((long long)M * K >= INT_MAX || (long long)M * N >= INT_MAX || (long long)K * N >= INT_MAX)
    return HSQ_E_INVAL;
  // The contraction kernels address the padded operand blobs through 32-bit
  // buffer resources: the int8 activation codes (rows padded to 16, K to
  // 128) and the int8 operand part of the packed residual (columns padded
  // to 16) must each stay below 2^32 bytes, or the resource size would wrap
  // and every load read 0.
  const long long kpad = (long long)padded_groups(K) * kGroup;
  if ((long long)ceil_div(M, kTile) * kTile * kpad >= (1LL << 32) ||
      (long long)ceil_div(N, kTile) * kTile * kpad >= (1LL << 32))
    return HSQ_E_INVAL;
  return HSQ_OK;
}

// The HIP error behind the last HSQ_E_HIP of this host thread.
thread_local hipError_t g_last_hip_error = hipSuccess;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return HSQ_OK;
  g_last_hip_error = e;
  return HSQ_E_HIP;
}

// HSQ_DEBUG set (and not "0") in the environment: a call that enqueued work
// waits for its stream and reports an asynchronous failure of its kernels
// as HSQ_E_HIP (hsq_last_hip_error names it) -- except while the stream is
// being captured into a graph, where waiting is not allowed.
bool debug_enabled() {
  const char *v = getenv("HSQ_DEBUG");
  return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

int debug_check(int st, void *stream) {
  if (st != HSQ_OK || !debug_enabled()) return st;
  hipStream_t s = (hipStream_t)stream;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t ce = hipStreamIsCapturing(s, &cs);
  if (ce != hipSuccess) return hip_status(ce);
  if (cs != hipStreamCaptureStatusNone) return st;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipGetLastError();
  return hip_status(e);
}

bool group_ok(int group) { return group == 64 || group == 128; }

// Calibration sizes: K a positive multiple of 64 up to kCalibMaxK (H is
// K x K fp32, up to 1 GiB); the Hessian's token x channel count below 2^30.
constexpr int kCalibMaxK = 16384;
constexpr long long kCalibMaxMK = 1LL << 30;

int calib_sizes(int K) {
  if (K < kGroup || K > kCalibMaxK) return HSQ_E_INVAL;
  if (K % kGroup != 0) return HSQ_E_SHAPE;
  return HSQ_OK;
}

size_t workspace_bytes(int M, int K, int N, int r, int batch, int group) {
  if (check_sizes(M, K, N, r, batch) != HSQ_OK || !group_ok(group) || K % group != 0) return 0;
  return plan_workspace(M, K, N, r, batch, group).total;
}

// Argument checks shared by every form of the linear.  `quant` / `contract`
// select which stage's pointers must be present.
int validate(const uint16_t *X, int M, int K, int N, int batch, int group,
             const uint16_t *lambda, const uint8_t *packed_w, const uint16_t *sw,
             const uint16_t *L1, const uint16_t *L2, int r, const uint16_t *bias, const void *Y,
             int y_dtype, const void *workspace, size_t ws_bytes, int *kernel, bool quant,
             bool contract, const int32_t *P, int m0, int mc, int n0, int nc) {
  int st = check_sizes(M, K, N, r, batch);
  if (st != HSQ_OK) return st;
  if (!group_ok(group)) return HSQ_E_INVAL;
  if (K % group != 0) return HSQ_E_SHAPE;
  const bool dump = P != nullptr;
  if (!workspace) return HSQ_E_INVAL;
  if (quant && (!X || !lambda || (r > 0 && !L1))) return HSQ_E_INVAL;
  if (contract && !packed_w) return HSQ_E_INVAL;
  if (contract && !dump && (!sw || !Y || (r > 0 && !L2))) return HSQ_E_INVAL;
  if (contract && !dump && y_dtype != HSQ_F32 && y_dtype != HSQ_BF16) return HSQ_E_INVAL;
  if (*kernel != HSQ_KERNEL_AUTO && *kernel != HSQ_KERNEL_TILED && *kernel != HSQ_KERNEL_SKINNY)
    return HSQ_E_INVAL;
  if (dump && (mc < 1 || nc < 1 || m0 < 0 || n0 < 0 || m0 + mc > M || n0 + nc > N))
    return HSQ_E_SHAPE;
  const void *ptrs[] = {X, lambda, packed_w, sw, L1, L2, bias, Y, workspace, P};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return HSQ_E_ALIGN;
  if (*kernel == HSQ_KERNEL_AUTO) *kernel = M <= kSkinnyMaxM ? HSQ_KERNEL_SKINNY : HSQ_KERNEL_TILED;
  if (*kernel == HSQ_KERNEL_SKINNY && M > kSkinnyMaxM) return HSQ_E_INVAL;
  if (ws_bytes < plan_workspace(M, K, N, r, batch, group).total) return HSQ_E_WORKSPACE;
  return HSQ_OK;
}

int quant_stage(const uint16_t *X, int M, int K, int N, int batch, int group,
                const uint16_t *lambda, const uint16_t *L1, int r, void *workspace, hipStream_t s,
                int aq = HSQ_AQ_SYMMETRIC, const uint16_t *pair_sw = nullptr) {
  const WsLayout L = plan_workspace(M, K, N, r, batch, group);
  char *ws = (char *)workspace;
  QuantArgs q{};
  q.X = X;
  q.lam = lambda;
  q.L1 = r > 0 ? L1 : nullptr;
  q.M = M; q.K = K; q.G = K / kGroup;
  q.bpg = L.bpg; q.SG = L.SG;
  q.r = r; q.batch = batch;
  q.kend = L.Gp * kGroup;
  q.qa = (int8_t *)(ws + L.qa_off);
  q.sxs = (uint16_t *)(ws + L.sxs_off);
  q.uw = (float *)(ws + L.uw_off);
  q.Gp = L.Gp; q.Mpad = L.Mpad; q.ucols = batch * r;
  q.asym = aq == HSQ_AQ_ASYMMETRIC;
  if (pair_sw != nullptr) {   // the tiled contraction's weight-scale pairs ride along
    q.sw = pair_sw;
    q.swp = (float4 *)(ws + L.swp_off);
    q.swG = L.G; q.swN = N; q.swr = L.swr; q.swnpad = L.npad;
  }
  return hip_status(launch_quant_tiles(q, s));
}

int contract_stage(int M, int K, int N, int batch, int group, const uint8_t *packed_w,
                   const uint16_t *sw, const uint16_t *L2, int r, const uint16_t *bias, void *Y,
                   int y_dtype, void *workspace, int kernel, hipStream_t s, int32_t *P, int m0,
                   int mc, int n0, int nc, int u_slices = -1, bool pairs_written = false) {
  const WsLayout L = plan_workspace(M, K, N, r, batch, group);
  char *ws = (char *)workspace;
  GemmArgs g{};
  g.qa = (const int8_t *)(ws + L.qa_off);
  g.sxs = (const uint16_t *)(ws + L.sxs_off);
  g.w = packed_w;
  g.w_stride = packed_bytes(K, N);
  g.w_ops = nibble_bytes(K, N);
  g.sw = sw;
  g.uw = (const float *)(ws + L.uw_off);
  g.u_slices = u_slices >= 0 ? u_slices : L.u_slices;
  g.L2 = r > 0 ? L2 : nullptr;
  g.bias = bias;
  g.Y = Y;
  g.y_bf16 = y_dtype == HSQ_BF16;
  g.M = M; g.N = N; g.G = L.G; g.Gp = L.Gp; g.Mpad = L.Mpad; g.r = r; g.ucols = batch * r;
  g.bpg = L.bpg; g.SG = L.SG;
  g.P = P; g.m0 = m0; g.mc = mc; g.n0 = n0; g.nc = nc;
  g.part = (float *)(ws + L.part_off);
  g.swp = (const float2 *)(ws + L.swp_off);
  g.swr = L.swr;
  g.npad = L.npad;
  const bool dump = P != nullptr;
  if (kernel == HSQ_KERNEL_SKINNY) return hip_status(launch_gemm_skinny(g, batch, dump, s));
  if (!dump && !pairs_written) {
    const hipError_t e = launch_sw_pairs(g, batch, s);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(launch_gemm_tiled(g, batch, dump, s));
}

int run_linear(const uint16_t *X, int M, int K, int N, int batch, int group,
               const uint16_t *lambda, const uint8_t *packed_w, const uint16_t *sw,
               const uint16_t *L1, const uint16_t *L2, int r, const uint16_t *bias, void *Y,
               int y_dtype, void *workspace, size_t ws_bytes, int kernel, void *stream,
               // partial-sum dump (test export); P == nullptr for the linear
               int32_t *P, int m0, int mc, int n0, int nc, int aq = HSQ_AQ_SYMMETRIC) {
  int st = validate(X, M, K, N, batch, group, lambda, packed_w, sw, L1, L2, r, bias, Y, y_dtype,
                    workspace, ws_bytes, &kernel, true, true, P, m0, mc, n0, nc);
  if (st != HSQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // the tiled contraction's weight-scale pairs are written by the
  // quantization pass's launch (no launch of their own)
  const bool pairs = kernel == HSQ_KERNEL_TILED && P == nullptr;
  st = quant_stage(X, M, K, N, batch, group, lambda, L1, r, workspace, s, aq, pairs ? sw : nullptr);
  if (st != HSQ_OK) return st;
  return contract_stage(M, K, N, batch, group, packed_w, sw, L2, r, bias, Y, y_dtype, workspace,
                        kernel, s, P, m0, mc, n0, nc, -1, pairs);
}

int quantize_stage_g(const uint16_t *X, int M, int K, int N, int batch, int group,
                     const uint16_t *lambda, const uint16_t *L1, int r, void *workspace,
                     size_t ws_bytes, void *stream, int aq = HSQ_AQ_SYMMETRIC) {
  int kernel = HSQ_KERNEL_AUTO;
  int st = validate(X, M, K, N, batch, group, lambda, nullptr, nullptr, L1, nullptr, r, nullptr,
                    nullptr, HSQ_F32, workspace, ws_bytes, &kernel, true, false, nullptr, 0, 0, 0, 0);
  if (st != HSQ_OK) return st;
  return quant_stage(X, M, K, N, batch, group, lambda, L1, r, workspace, (hipStream_t)stream, aq);
}

int contract_stage_g(int M, int K, int N, int batch, int group, const uint8_t *packed_w,
                     const uint16_t *sw, const uint16_t *L2, int r, const uint16_t *bias, void *Y,
                     int y_dtype, void *workspace, size_t ws_bytes, int kernel, void *stream) {
  int st = validate(nullptr, M, K, N, batch, group, nullptr, packed_w, sw, nullptr, L2, r, bias, Y,
                    y_dtype, workspace, ws_bytes, &kernel, false, true, nullptr, 0, 0, 0, 0);
  if (st != HSQ_OK) return st;
  return contract_stage(M, K, N, batch, group, packed_w, sw, L2, r, bias, Y, y_dtype, workspace,
                        kernel, (hipStream_t)stream, nullptr, 0, 0, 0, 0);
}

// Fused two-layer chain (group 64, one projection each): workspace of the
// up layer, of the down layer, and the down layer's U shares per 128-column
// block of the hidden width.
struct ChainLayout {
  WsLayout up, dn;
  size_t up_off = 0, dn_off = 0, upart_off = 0, total = 0;
  int nblk = 0;
};

ChainLayout plan_chain(int M, int K, int H, int N, int r1, int r2) {
  ChainLayout c;
  c.up = plan_workspace(M, K, H, r1, 1, kGroup);
  c.dn = plan_workspace(M, H, N, r2, 1, kGroup);
  c.nblk = ceil_div(H, 128);
  c.up_off = 0;
  c.dn_off = align_up(c.up.total, 256);
  c.upart_off = align_up(c.dn_off + c.dn.total, 256);
  c.total = align_up(c.upart_off + (size_t)c.nblk * r2 * c.up.Mpad * sizeof(float), 256);
  return c;
}

int chain_sizes(int M, int K, int H, int N, int r1, int r2) {
  int st = check_sizes(M, K, H, r1, 1);
  if (st != HSQ_OK) return st;
  st = check_sizes(M, H, N, r2, 1);
  if (st != HSQ_OK) return st;
  if (r2 > kChainMaxRank) return HSQ_E_INVAL;
  return HSQ_OK;
}

int run_chain(const uint16_t *X, int M, int K, int H, int N, const uint16_t *lam_up,
              const uint8_t *packed_up, const uint16_t *sw_up, const uint16_t *L1_up,
              const uint16_t *L2_up, int r1, const uint16_t *bias_up, int act,
              const uint16_t *lam_dn, const uint8_t *packed_dn, const uint16_t *sw_dn,
              const uint16_t *L1_dn, const uint16_t *L2_dn, int r2, const uint16_t *bias_dn, void *Y,
              int y_dtype, float *yhid, void *workspace, size_t ws_bytes, void *stream) {
  int st = chain_sizes(M, K, H, N, r1, r2);
  if (st != HSQ_OK) return st;
  if (act != HSQ_ACT_IDENTITY && act != HSQ_ACT_GELU_TANH) return HSQ_E_INVAL;
  if (y_dtype != HSQ_F32 && y_dtype != HSQ_BF16) return HSQ_E_INVAL;
  if (!X || !lam_up || !packed_up || !sw_up || !lam_dn || !packed_dn || !sw_dn || !Y || !workspace)
    return HSQ_E_INVAL;
  if ((r1 > 0 && (!L1_up || !L2_up)) || (r2 > 0 && (!L1_dn || !L2_dn))) return HSQ_E_INVAL;
  const void *ptrs[] = {X, lam_up, packed_up, sw_up, L1_up, L2_up, bias_up, lam_dn, packed_dn,
                        sw_dn, L1_dn, L2_dn, bias_dn, Y, yhid, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return HSQ_E_ALIGN;
  const ChainLayout c = plan_chain(M, K, H, N, r1, r2);
  if (ws_bytes < c.total) return HSQ_E_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  char *wup = ws + c.up_off, *wdn = ws + c.dn_off;
  // 1. the up layer's quantization pass (with its contraction's weight-scale
  //    pairs)
  st = quant_stage(X, M, K, H, 1, kGroup, lam_up, L1_up, r1, wup, s, HSQ_AQ_SYMMETRIC, sw_up);
  if (st != HSQ_OK) return st;
  // 2. its contraction, whose epilogue quantizes act(Y) into the down
  //    layer's workspace
  GemmArgs g{};
  g.qa = (const int8_t *)(wup + c.up.qa_off);
  g.sxs = (const uint16_t *)(wup + c.up.sxs_off);
  g.w = packed_up;
  g.w_stride = packed_bytes(K, H);
  g.w_ops = nibble_bytes(K, H);
  g.sw = sw_up;
  g.uw = (const float *)(wup + c.up.uw_off);
  g.u_slices = c.up.u_slices;
  g.L2 = r1 > 0 ? L2_up : nullptr;
  g.bias = bias_up;
  g.M = M; g.N = H; g.G = c.up.G; g.Gp = c.up.Gp; g.Mpad = c.up.Mpad; g.r = r1; g.ucols = r1;
  g.bpg = 1; g.SG = c.up.SG;
  g.splits = 1;
  g.act = act;
  g.lam2 = lam_dn;
  g.L1n = r2 > 0 ? L1_dn : nullptr;
  g.r2 = r2;
  g.Gp2 = c.dn.Gp;
  g.qa2 = (int8_t *)(wdn + c.dn.qa_off);
  g.sxs2 = (uint16_t *)(wdn + c.dn.sxs_off);
  g.upart2 = (float *)(ws + c.upart_off);
  g.yhid = yhid;
  g.swp = (const float2 *)(wup + c.up.swp_off);
  g.swr = c.up.swr;
  g.npad = c.up.npad;
  st = hip_status(launch_gemm_tiled_chain(g, s));
  if (st != HSQ_OK) return st;
  // 3. the down layer's U: the column-block shares summed in order
  if (r2 > 0) {
    st = hip_status(launch_chain_ureduce(g.upart2, c.nblk, r2, c.up.Mpad, (float *)(wdn + c.dn.uw_off), s));
    if (st != HSQ_OK) return st;
  }
  // 4. the down layer's contraction from that workspace (one U slice)
  const int kernel = M <= kSkinnyMaxM ? HSQ_KERNEL_SKINNY : HSQ_KERNEL_TILED;
  return contract_stage(M, H, N, 1, kGroup, packed_dn, sw_dn, L2_dn, r2, bias_dn, Y, y_dtype, wdn,
                        kernel, s, nullptr, 0, 0, 0, 0, 1);
}

int group_partials_g(const uint16_t *X, int M, int K, int N, int group, const uint16_t *lambda,
                     const uint8_t *packed_w, int m0, int mc, int n0, int nc, int32_t *P,
                     void *workspace, size_t ws_bytes, int kernel, void *stream,
                     int aq = HSQ_AQ_SYMMETRIC) {
  if (!P) return HSQ_E_INVAL;
  return run_linear(X, M, K, N, 1, group, lambda, packed_w, nullptr, nullptr, nullptr, 0, nullptr,
                    nullptr, HSQ_F32, workspace, ws_bytes, kernel, stream, P, m0, mc, n0, nc, aq);
}

bool aq_ok(int aq) { return aq == HSQ_AQ_SYMMETRIC || aq == HSQ_AQ_ASYMMETRIC; }

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch of hsq_w4a4_lowrank_linear_noalloc: the layer's workspace in
// a device array of fixed size, for callers that cannot allocate.  Every GPU
// the library runs on holds its own copy of it until the process ends.  In
// host code `scratch` only names the symbol: its device address on the
// current GPU comes from hipGetSymbolAddress (once per device, on the first
// no-alloc call with that device current) and only that address is passed
// to the kernels.
static __device__ __align__(256) unsigned char scratch[HSQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array.
int scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return HSQ_E_INVAL;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      if (!p) return HSQ_E_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return HSQ_OK;
}

}  // namespace

extern "C" {

int hsq_layout_version(void) { return 2; }

const char *hsq_status_string(int status) {
  switch (status) {
    case HSQ_OK: return "ok";
    case HSQ_E_INVAL: return "invalid argument";
    case HSQ_E_SHAPE: return "invalid shape (K must be a positive multiple of 64; window inside the matrix)";
    case HSQ_E_ALIGN: return "pointer not 16-byte aligned";
    case HSQ_E_WORKSPACE: return "workspace missing or too small";
    case HSQ_E_HIP: return "HIP launch failed";
    case HSQ_E_SCRATCH: return "the sizes need more workspace than the no-alloc entry point's static scratch holds";
    default: return "unknown status";
  }
}

const char *hsq_last_hip_error(void) {
  return g_last_hip_error == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip_error);
}

size_t hsq_packed_weight_bytes(int K, int N) {
  if (K < kGroup || K % kGroup != 0 || N < 1 || (long long)K * N >= INT_MAX) return 0;
  return packed_bytes(K, N);
}

int hsq_pack_weights(const int8_t *codes, int K, int N, uint8_t *packed, int *d_status,
                     void *stream) {
  if (!codes || !packed || !d_status || N < 1 || K < 1) return HSQ_E_INVAL;
  if (K % kGroup != 0) return HSQ_E_SHAPE;
  if ((long long)K * N >= INT_MAX) return HSQ_E_INVAL;
  if (!aligned16(codes) || !aligned16(packed) || !aligned16(d_status)) return HSQ_E_ALIGN;
  return debug_check(hip_status(launch_pack(codes, K, N, packed, d_status, (hipStream_t)stream)), stream);
}

int hsq_unpack_weights(const uint8_t *packed, int K, int N, int8_t *codes, void *stream) {
  if (!codes || !packed || N < 1 || K < 1) return HSQ_E_INVAL;
  if (K % kGroup != 0) return HSQ_E_SHAPE;
  if ((long long)K * N >= INT_MAX) return HSQ_E_INVAL;
  if (!aligned16(codes) || !aligned16(packed)) return HSQ_E_ALIGN;
  return debug_check(hip_status(launch_unpack(packed, K, N, codes, (hipStream_t)stream)), stream);
}

int hsq_quantize_act(const uint16_t *X, int M, int K, const uint16_t *lambda,
                     const uint16_t *L1, int r, uint8_t *qx, uint16_t *sx, float *U,
                     void *stream) {
  int st = check_sizes(M, K, 1, r, 1);
  if (st != HSQ_OK) return st;
  if (K > kQuantActMaxK) return HSQ_E_INVAL;
  if (!X || !lambda || !qx || !sx || (r > 0 && (!L1 || !U))) return HSQ_E_INVAL;
  const void *ptrs[] = {X, lambda, L1, qx, sx, U};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return HSQ_E_ALIGN;
  QuantArgs q{};
  q.X = X;
  q.lam = lambda;
  q.L1 = r > 0 ? L1 : nullptr;
  q.M = M; q.K = K; q.G = K / kGroup;
  q.r = r; q.batch = 1;
  q.kend = K;
  q.qx = qx; q.sx = sx; q.u_pub = r > 0 ? U : nullptr;
  q.ucols = r;
  return debug_check(hip_status(launch_quant_act(q, (hipStream_t)stream)), stream);
}

size_t hsq_workspace_bytes(int M, int K, int N, int r, int batch) {
  return workspace_bytes(M, K, N, r, batch, kGroup);
}

size_t hsq_workspace_bytes_g(int M, int K, int N, int r, int batch, int group) {
  return workspace_bytes(M, K, N, r, batch, group);
}

int hsq_w4a4_lowrank_linear(const uint16_t *X, int M, int K, int N, int batch,
                            const uint16_t *lambda, const uint8_t *packed_w,
                            const uint16_t *sw, const uint16_t *L1, const uint16_t *L2, int r,
                            const uint16_t *bias, void *Y, int y_dtype, void *workspace,
                            size_t ws_bytes, void *stream) {
  return debug_check(run_linear(X, M, K, N, batch, kGroup, lambda, packed_w, sw, L1, L2, r, bias, Y, y_dtype,
                    workspace, ws_bytes, HSQ_KERNEL_AUTO, stream, nullptr, 0, 0, 0, 0), stream);
}

int hsq_w4a4_lowrank_linear_noalloc(const uint16_t *X, int M, int K, int N, int batch,
                                    const uint16_t *lambda, const uint8_t *packed_w,
                                    const uint16_t *sw, const uint16_t *L1, const uint16_t *L2,
                                    int r, const uint16_t *bias, void *Y, int y_dtype,
                                    void *stream) {
  // every argument is checked before any device call: sizes, the bound of
  // the static scratch, then the pointers (with an aligned placeholder in
  // the workspace's place); only then is the scratch's address looked up
  int st = check_sizes(M, K, N, r, batch);
  if (st != HSQ_OK) return st;
  if (plan_workspace(M, K, N, r, batch, kGroup).total > (size_t)HSQ_NOALLOC_SCRATCH_BYTES)
    return HSQ_E_SCRATCH;
  int kernel = HSQ_KERNEL_AUTO;
  void *const placeholder = reinterpret_cast<void *>((uintptr_t)256);
  st = validate(X, M, K, N, batch, kGroup, lambda, packed_w, sw, L1, L2, r, bias, Y, y_dtype, placeholder,
                (size_t)HSQ_NOALLOC_SCRATCH_BYTES, &kernel, true, true, nullptr, 0, 0, 0, 0);
  if (st != HSQ_OK) return st;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != HSQ_OK) return st;
  return debug_check(run_linear(X, M, K, N, batch, kGroup, lambda, packed_w, sw, L1, L2, r, bias, Y, y_dtype, ws,
                    (size_t)HSQ_NOALLOC_SCRATCH_BYTES, HSQ_KERNEL_AUTO, stream, nullptr, 0, 0, 0, 0), stream);
}

int hsq_w4a4_lowrank_linear_ex(const uint16_t *X, int M, int K, int N, int batch,
                               const uint16_t *lambda, const uint8_t *packed_w,
                               const uint16_t *sw, const uint16_t *L1, const uint16_t *L2,
                               int r, const uint16_t *bias, void *Y, int y_dtype,
                               void *workspace, size_t ws_bytes, int kernel, void *stream) {
  return debug_check(run_linear(X, M, K, N, batch, kGroup, lambda, packed_w, sw, L1, L2, r, bias, Y, y_dtype,
                    workspace, ws_bytes, kernel, stream, nullptr, 0, 0, 0, 0), stream);
}

int hsq_w4a4_lowrank_linear_g(const uint16_t *X, int M, int K, int N, int batch, int group,
                              const uint16_t *lambda, const uint8_t *packed_w,
                              const uint16_t *sw, const uint16_t *L1, const uint16_t *L2,
                              int r, const uint16_t *bias, void *Y, int y_dtype,
                              void *workspace, size_t ws_bytes, int kernel, void *stream) {
  return debug_check(run_linear(X, M, K, N, batch, group, lambda, packed_w, sw, L1, L2, r, bias, Y, y_dtype,
                    workspace, ws_bytes, kernel, stream, nullptr, 0, 0, 0, 0), stream);
}

int hsq_w4a4_quantize_stage(const uint16_t *X, int M, int K, int N, int batch,
                            const uint16_t *lambda, const uint16_t *L1, int r, void *workspace,
                            size_t ws_bytes, void *stream) {
  return debug_check(quantize_stage_g(X, M, K, N, batch, kGroup, lambda, L1, r, workspace, ws_bytes, stream), stream);
}

int hsq_w4a4_quantize_stage_g(const uint16_t *X, int M, int K, int N, int batch, int group,
                              const uint16_t *lambda, const uint16_t *L1, int r, void *workspace,
                              size_t ws_bytes, void *stream) {
  return debug_check(quantize_stage_g(X, M, K, N, batch, group, lambda, L1, r, workspace, ws_bytes, stream), stream);
}

int hsq_w4a4_contract_stage(int M, int K, int N, int batch, const uint8_t *packed_w,
                            const uint16_t *sw, const uint16_t *L2, int r, const uint16_t *bias,
                            void *Y, int y_dtype, void *workspace, size_t ws_bytes, int kernel,
                            void *stream) {
  return debug_check(contract_stage_g(M, K, N, batch, kGroup, packed_w, sw, L2, r, bias, Y, y_dtype, workspace,
                          ws_bytes, kernel, stream), stream);
}

int hsq_w4a4_contract_stage_g(int M, int K, int N, int batch, int group, const uint8_t *packed_w,
                              const uint16_t *sw, const uint16_t *L2, int r, const uint16_t *bias,
                              void *Y, int y_dtype, void *workspace, size_t ws_bytes, int kernel,
                              void *stream) {
  return debug_check(contract_stage_g(M, K, N, batch, group, packed_w, sw, L2, r, bias, Y, y_dtype, workspace,
                          ws_bytes, kernel, stream), stream);
}

int hsq_w4a4_group_partials(const uint16_t *X, int M, int K, int N, const uint16_t *lambda,
                            const uint8_t *packed_w, int m0, int mc, int n0, int nc,
                            int32_t *P, void *workspace, size_t ws_bytes, int kernel,
                            void *stream) {
  return debug_check(group_partials_g(X, M, K, N, kGroup, lambda, packed_w, m0, mc, n0, nc, P, workspace,
                          ws_bytes, kernel, stream), stream);
}

int hsq_w4a4_group_partials_g(const uint16_t *X, int M, int K, int N, int group,
                              const uint16_t *lambda, const uint8_t *packed_w, int m0, int mc,
                              int n0, int nc, int32_t *P, void *workspace, size_t ws_bytes,
                              int kernel, void *stream) {
  return debug_check(group_partials_g(X, M, K, N, group, lambda, packed_w, m0, mc, n0, nc, P, workspace,
                          ws_bytes, kernel, stream), stream);
}

int hsq_w4a4_lowrank_linear_aq(const uint16_t *X, int M, int K, int N, int batch, int group,
                               int act_quant, const uint16_t *lambda, const uint8_t *packed_w,
                               const uint16_t *sw, const uint16_t *L1, const uint16_t *L2, int r,
                               const uint16_t *bias, void *Y, int y_dtype, void *workspace,
                               size_t ws_bytes, int kernel, void *stream) {
  if (!aq_ok(act_quant)) return HSQ_E_INVAL;
  return debug_check(run_linear(X, M, K, N, batch, group, lambda, packed_w, sw, L1, L2, r, bias, Y, y_dtype,
                    workspace, ws_bytes, kernel, stream, nullptr, 0, 0, 0, 0, act_quant), stream);
}

int hsq_w4a4_quantize_stage_aq(const uint16_t *X, int M, int K, int N, int batch, int group,
                               int act_quant, const uint16_t *lambda, const uint16_t *L1, int r,
                               void *workspace, size_t ws_bytes, void *stream) {
  if (!aq_ok(act_quant)) return HSQ_E_INVAL;
  return debug_check(quantize_stage_g(X, M, K, N, batch, group, lambda, L1, r, workspace, ws_bytes, stream,
                          act_quant), stream);
}

int hsq_w4a4_group_partials_aq(const uint16_t *X, int M, int K, int N, int group, int act_quant,
                               const uint16_t *lambda, const uint8_t *packed_w, int m0, int mc,
                               int n0, int nc, int32_t *P, void *workspace, size_t ws_bytes,
                               int kernel, void *stream) {
  if (!aq_ok(act_quant)) return HSQ_E_INVAL;
  return debug_check(group_partials_g(X, M, K, N, group, lambda, packed_w, m0, mc, n0, nc, P, workspace,
                          ws_bytes, kernel, stream, act_quant), stream);
}

// ---------------------------------------------------------------- MX-fp4 variant

size_t hsq_mx_packed_weight_bytes(int K, int N) {
  if (K < kGroup || K % kGroup != 0 || N < 1 || (long long)K * N >= INT_MAX) return 0;
  return mx_packed_bytes(K, N);
}

int hsq_mx_pack_weights(const float *R, int K, int N, uint8_t *packed, void *stream) {
  if (!R || !packed || N < 1 || K < 1) return HSQ_E_INVAL;
  if (K % kGroup != 0) return HSQ_E_SHAPE;
  if ((long long)K * N >= INT_MAX) return HSQ_E_INVAL;
  if (!aligned16(R) || !aligned16(packed)) return HSQ_E_ALIGN;
  return debug_check(hip_status(launch_mx_pack(R, K, N, packed, (hipStream_t)stream)), stream);
}

size_t hsq_mx_workspace_bytes(int M, int K, int r) {
  if (check_sizes(M, K, 1, r, 1) != HSQ_OK) return 0;
  return plan_mx(M, K, r).total;
}

int hsq_mx_lowrank_linear(const uint16_t *X, int M, int K, int N, const uint16_t *lambda,
                          const uint8_t *packed_mx, const uint16_t *L1, const uint16_t *L2, int r,
                          const uint16_t *bias, void *Y, int y_dtype, void *workspace, size_t ws_bytes,
                          void *stream) {
  int st = check_sizes(M, K, N, r, 1);
  if (st != HSQ_OK) return st;
  if (!X || !lambda || !packed_mx || !Y || !workspace || (r > 0 && (!L1 || !L2))) return HSQ_E_INVAL;
  if (y_dtype != HSQ_F32 && y_dtype != HSQ_BF16) return HSQ_E_INVAL;
  const void *ptrs[] = {X, lambda, packed_mx, L1, L2, bias, Y, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return HSQ_E_ALIGN;
  const MxLayout L = plan_mx(M, K, r);
  if (ws_bytes < L.total) return HSQ_E_WORKSPACE;
  char *ws = (char *)workspace;
  MxArgs a{};
  a.X = X; a.lam = lambda; a.L1 = r > 0 ? L1 : nullptr; a.L2 = r > 0 ? L2 : nullptr; a.bias = bias;
  a.qa = (uint8_t *)(ws + L.qa_off);
  a.sa = (uint8_t *)(ws + L.sa_off);
  a.U = (float *)(ws + L.u_off);
  a.wq = packed_mx;
  a.ws = packed_mx + (size_t)ceil_div(N, 16) * L.KS * 1024;
  a.Y = Y; a.y_bf16 = y_dtype == HSQ_BF16;
  a.M = M; a.K = K; a.N = N; a.r = r; a.KS = L.KS; a.KS4 = L.KS4; a.Mpad = L.Mpad;
  a.u_slices = L.KS4;
  return debug_check(hip_status(launch_mx_linear(a, (hipStream_t)stream)), stream);
}

// ---------------------------------------------------------------- fused chain

size_t hsq_mlp_workspace_bytes(int M, int K, int H, int N, int r1, int r2) {
  if (chain_sizes(M, K, H, N, r1, r2) != HSQ_OK) return 0;
  return plan_chain(M, K, H, N, r1, r2).total;
}

int hsq_w4a4_lowrank_mlp(const uint16_t *X, int M, int K, int H, int N, const uint16_t *lambda_up,
                         const uint8_t *packed_up, const uint16_t *sw_up, const uint16_t *L1_up,
                         const uint16_t *L2_up, int r_up, const uint16_t *bias_up, int act,
                         const uint16_t *lambda_down, const uint8_t *packed_down,
                         const uint16_t *sw_down, const uint16_t *L1_down, const uint16_t *L2_down,
                         int r_down, const uint16_t *bias_down, void *Y, int y_dtype, float *Y_hidden,
                         void *workspace, size_t ws_bytes, void *stream) {
  return debug_check(run_chain(X, M, K, H, N, lambda_up, packed_up, sw_up, L1_up, L2_up, r_up, bias_up, act,
                   lambda_down, packed_down, sw_down, L1_down, L2_down, r_down, bias_down, Y, y_dtype,
                   Y_hidden, workspace, ws_bytes, stream), stream);
}

// ---------------------------------------------------------------- calibration

size_t hsq_hessian_workspace_bytes(int M, int K) {
  if (calib_sizes(K) != HSQ_OK || M < 1 || (long long)M * K >= kCalibMaxMK) return 0;
  return hessian_workspace_bytes(M, K);
}

int hsq_hessian_accumulate(const uint16_t *X, int M, int K, const uint16_t *lambda, float *H,
                           int accumulate, void *workspace, size_t ws_bytes, void *stream) {
  int st = calib_sizes(K);
  if (st != HSQ_OK) return st;
  if (M < 1 || (long long)M * K >= kCalibMaxMK || (accumulate != 0 && accumulate != 1)) return HSQ_E_INVAL;
  if (!X || !lambda || !H) return HSQ_E_INVAL;
  const void *ptrs[] = {X, lambda, H, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return HSQ_E_ALIGN;
  const size_t need = hessian_workspace_bytes(M, K);
  if (need > 0 && (!workspace || ws_bytes < need)) return HSQ_E_WORKSPACE;
  HessArgs a{};
  a.X = X; a.lam = lambda; a.H = H; a.M = M; a.K = K; a.accumulate = accumulate;
  a.part = (float *)workspace;
  return debug_check(hip_status(launch_hessian(a, (hipStream_t)stream)), stream);
}

size_t hsq_deflate_workspace_bytes(int K, int r) {
  if (calib_sizes(K) != HSQ_OK || r < 1 || r > kMaxRank) return 0;
  return deflate_workspace_bytes(K, r);
}

int hsq_deflate_hessian(const float *H, int K, const uint16_t *L1, int r, float *Hperp, float *HL1,
                        double *Cinv, void *workspace, size_t ws_bytes, void *stream) {
  int st = calib_sizes(K);
  if (st != HSQ_OK) return st;
  if (r < 1 || r > kMaxRank || !H || !L1 || !Hperp || !HL1 || !Cinv || !workspace) return HSQ_E_INVAL;
  const void *ptrs[] = {H, L1, Hperp, HL1, Cinv, workspace};
  for (const void *p : ptrs)
    if (!aligned16(p)) return HSQ_E_ALIGN;
  if (ws_bytes < deflate_workspace_bytes(K, r)) return HSQ_E_WORKSPACE;
  DeflArgs a{};
  a.H = H; a.Hperp = Hperp; a.L1 = L1; a.HL1 = HL1; a.Cinv = Cinv; a.K = K; a.r = r;
  a.L1f = (float *)workspace;
  a.Cpart = (double *)((char *)workspace + align_up((size_t)K * rank_pad(r) * sizeof(float), 256));
  return debug_check(hip_status(launch_deflate(a, (hipStream_t)stream)), stream);
}

size_t hsq_closed_form_l2_workspace_bytes(int K, int N, int r) {
  if (calib_sizes(K) != HSQ_OK || r < 1 || r > kMaxRank || N < 1 || (long long)K * N >= INT_MAX) return 0;
  return l2_workspace_bytes(K, N, r);
}

int hsq_closed_form_l2(const float *HL1, const double *Cinv, int K, int N, int r, int group,
                       const uint16_t *W, const uint8_t *packed_w, const uint16_t *sw, float *L2,
                       void *workspace, size_t ws_bytes, void *stream) {
  int st = calib_sizes(K);
  if (st != HSQ_OK) return st;
  if (!group_ok(group)) return HSQ_E_INVAL;
  if (K % group != 0) return HSQ_E_SHAPE;
  if (r < 1 || r > kMaxRank || N < 1 || (long long)K * N >= INT_MAX) return HSQ_E_INVAL;
  if (!HL1 || !Cinv || !W || !packed_w || !sw || !L2 || !workspace) return HSQ_E_INVAL;
  const void *ptrs[] = {HL1, Cinv, W, packed_w, sw, L2, workspace};
  for (const void *p : ptrs)
    if (!aligned16(p)) return HSQ_E_ALIGN;
  if (ws_bytes < l2_workspace_bytes(K, N, r)) return HSQ_E_WORKSPACE;
  L2Args a{};
  a.HL1 = HL1; a.Cinv = Cinv; a.W = W; a.packed = packed_w; a.sw = sw; a.L2 = L2;
  a.Tpart = (float *)workspace;
  a.K = K; a.N = N; a.r = r; a.group = group;
  return debug_check(hip_status(launch_l2(a, (hipStream_t)stream)), stream);
}

}  // extern "C"

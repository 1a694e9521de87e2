// hsq_internal.h -- internal declarations shared by the libhsq translation
// units: data layouts in HBM, kernel argument blocks, launch entry points and
// small device helpers.  Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace hsq {

constexpr int kGroup = 64;       // input channels per quantization group
constexpr int kTile = 16;        // rows / columns per MFMA tile (16x16x64 i8)
constexpr int kMaxRank = 32;     // largest rank r of the high-precision branch
constexpr int kMaxBatch = 16;    // projections sharing one input
constexpr int kRankBlock = 32;   // rank columns one quantization pass accumulates
constexpr int kMaxUSlices = 8;   // U slices the contraction kernels prefetch (more: summed in a loop)
constexpr int kMaxSliceGroups = 192;  // groups per workgroup of the quantization pass (LDS)
constexpr int kQuantActMaxK = kMaxSliceGroups * kGroup;  // hsq_quantize_act: one slice

// Bits of the float 1.5 * 2^23: adding an integer n (|n| < 2^22) to these
// bits gives the float 1.5 * 2^23 + n exactly.  The contraction kernels feed
// it as the MFMA accumulator input so that the int32 result is read as a
// float without a conversion instruction.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Packed residual layout (hsq_pack_weights).  With NT = ceil(N/16) column
// tiles and Gp = G rounded up to even, the blob is NT x (Gp/2) blocks of
// 1024 bytes.  Block (nt, gp) holds 64 lane slots of 16 bytes; slot l
// serves output column 16*nt + l%16 and, for both groups g = 2gp + h
// (h = 0: bytes 0-7, h = 1: bytes 8-15), the 16 input channels
// k = 64g + 16*(l/16) + p, p = 0..15, as nibbles:
//   byte b in 0..3 : high nibble p = b,      low nibble p = b + 4
//   byte b in 4..7 : high nibble p = b + 4,  low nibble p = b + 8
// so that (w & 0xF0F0F0F0) and ((w << 4) & 0xF0F0F0F0) of the two little-
// endian dwords give the 16 int8 MFMA operand bytes 16*code in order p.
// ---------------------------------------------------------------------------
inline int padded_groups(int K) { return ceil_div(K / kGroup, 2) * 2; }
// Scale groups of `group` channels (64 or 128): one scale per (row or
// column, group).  A group-128 scale covers two 64-channel blocks, which is
// one block pair of the packed residual.  The activation scales are stored
// per row tile for every padded 64-block (group 64) or every group (128).
inline int scale_groups_stored(int K, int group) { return group == kGroup ? padded_groups(K) : K / group; }
inline size_t packed_bytes(int K, int N) {
  return (size_t)ceil_div(N, kTile) * (size_t)(padded_groups(K) / 2) * 1024u;
}

// ---------------------------------------------------------------------------
// Workspace of the fused linear.  MT = ceil(M/16) row tiles.
//   qa  : MT x Gp x 64 lanes x 16 int8 codes   (MFMA A-operand order:
//         lane l of block (mt, g) holds row 16mt + l%16, channels
//         64g + 16(l/16) + p, p = 0..15; pad rows / groups are zero)
//   sxs : MT x SG x 16 fp16, the activation scale of (row, scale group),
//         zero for pad rows / groups (read straight into v_fma_mix_f32);
//         SG = scale_groups_stored(K, group)
//   uw  : S_u x (batch*r) x (16*MT) fp32, one slice of U per K-slice of the
//         quantization pass, summed in slice order by the consumer
//   part: split-K partial tiles of the tiled contraction when its grid is
//         too small for the chip (tiled_partial_bytes; empty otherwise)
// ---------------------------------------------------------------------------
struct WsLayout {
  int MT = 0, G = 0, Gp = 0, Mpad = 0;
  int group = kGroup, bpg = 1, SG = 0;  // G = K/group scale groups; bpg = group/64 blocks each
  int u_slices = 0;      // S_u: K-slices of the quantization pass
  size_t qa_off = 0, sxs_off = 0, uw_off = 0, part_off = 0, total = 0;
};

// Plans the workspace for (M, K, N, r, batch, group).  Pure host arithmetic.
WsLayout plan_workspace(int M, int K, int N, int r, int batch, int group);

// Largest token count the skinny kernel accepts (4 row tiles).
constexpr int kSkinnyMaxM = 64;

// ---------------------------------------------------------------------------
// Kernel argument blocks
// ---------------------------------------------------------------------------
struct QuantArgs {
  const uint16_t *X;       // M x K bf16
  const uint16_t *lam;     // K fp16
  const uint16_t *L1;      // batch x K x r bf16 (or null)
  int M, K, G;             // G = K/64 real 64-channel blocks
  int bpg, SG;             // blocks per scale group (1 or 2); scale groups stored per row tile
  int r, batch;
  int c0, cb;              // rank columns [c0, c0 + cb) of the batch*r columns
  int kend;                // channels processed: K (public) or 64*Gp (internal)
  int write_codes;         // 0: rank pass only
  // public outputs (packed codes, fp16 scales, U as M x r)
  uint8_t *qx;
  uint16_t *sx;
  float *u_pub;
  // internal outputs (tiled codes, fp32 scales / 16, U slices)
  int8_t *qa;
  uint16_t *sxs;
  float *uw;
  int Gp, Mpad, ucols;
};

struct GemmArgs {
  const int8_t *qa;
  const uint16_t *sxs;
  const uint8_t *w;        // packed residual of projection 0
  size_t w_stride;         // bytes between projections
  const uint16_t *sw;      // batch x G x N fp16
  const float *uw;         // U slices (see WsLayout)
  int u_slices;
  const uint16_t *L2;      // batch x r x N bf16
  const uint16_t *bias;    // batch x N bf16 or null
  void *Y;                 // batch x M x N
  int y_bf16;
  int M, N, G, Gp, Mpad, r, ucols;  // G = K/group scale groups; Gp = padded 64-blocks
  int bpg, SG;             // blocks per scale group (1 or 2); scale groups stored per row tile
  // partial-sum dump window (test export)
  int32_t *P;
  int m0, mc, n0, nc;
  // split-K partial tiles of the tiled contraction (workspace) and their
  // number per output tile
  float *part;
  int splits;
};

hipError_t launch_pack(const int8_t *codes, int K, int N, uint8_t *packed, int *status,
                       hipStream_t s);
hipError_t launch_unpack(const uint8_t *packed, int K, int N, int8_t *codes, hipStream_t s);
// Quantization passes: the public layout (hsq_quantize_act, batch 1) and the
// fused linear's internal layout; each plans its own grid.  quant_slices()
// is the number of K-slices (U partials) of the internal pass.
hipError_t launch_quant_act(const QuantArgs &a, hipStream_t s);
hipError_t launch_quant_tiles(const QuantArgs &a, hipStream_t s);
int quant_slices(int M, int K, int r, int batch, int group);
hipError_t launch_gemm_tiled(const GemmArgs &a, int batch, bool dump, hipStream_t s);
// Split-K factor of the tiled contraction for this shape (1: no split) and
// the workspace bytes of its partial tiles.
int tiled_splits(int M, int N, int K, int batch, int group);
size_t tiled_partial_bytes(int M, int N, int K, int batch, int group);
hipError_t launch_gemm_skinny(const GemmArgs &a, int batch, bool dump, hipStream_t s);

// ---------------------------------------------------------------------------
// Calibration (calib.hip)
// ---------------------------------------------------------------------------
struct HessArgs {
  const uint16_t *X;       // M x K bf16 calibration activations (row-major)
  const uint16_t *lam;     // K fp16 smoothing factors
  float *H;                // K x K fp32
  int M, K;
  int accumulate;          // 0: H = Xh^T Xh; 1: H += Xh^T Xh
  float *part;             // token-split partial blocks (workspace)
  int splits;
};

struct DeflArgs {
  const float *H;          // K x K fp32
  float *Hperp;            // K x K fp32 (may equal H)
  const uint16_t *L1;      // K x r bf16
  float *HL1;              // K x r fp32 (output)
  double *Cinv;            // r x r fp64 (output)
  float *L1f;              // workspace: K x RP fp32, L1 padded to the rank template
  double *Cpart;           // workspace: per-workgroup shares of C
  int K, r;
};

struct L2Args {
  const float *HL1;        // K x r fp32
  const double *Cinv;      // r x r fp64
  const uint16_t *W;       // K x N bf16 full-precision (smoothed) weight
  const uint8_t *packed;   // packed residual codes of W's quantized residual
  const uint16_t *sw;      // (K / group) x N fp16 residual scales
  float *L2;               // r x N fp32 (output)
  float *Tpart;            // workspace: slices x r x N fp32
  int K, N, r, group;
};

int rank_pad(int r);
int hessian_splits(int M, int K);
size_t hessian_workspace_bytes(int M, int K);
hipError_t launch_hessian(const HessArgs &a, hipStream_t s);
int deflate_hl1_wgs(int K);
size_t deflate_workspace_bytes(int K, int r);
hipError_t launch_deflate(const DeflArgs &a, hipStream_t s);
int l2_slices(int K, int N, int r);
size_t l2_workspace_bytes(int K, int N, int r);
hipError_t launch_l2(const L2Args &a, hipStream_t s);

}  // namespace hsq

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#ifdef __HIPCC__
namespace hsq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Buffer resource over `bytes` bytes at p (raw, untyped; reads past the end
// return zero).  Loads through it take a 32-bit per-lane offset plus a
// uniform scalar offset, so loop-carried addressing costs no VALU.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Round to nearest even (v_cvt_f16_f32 in the default rounding mode).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace hsq
#endif

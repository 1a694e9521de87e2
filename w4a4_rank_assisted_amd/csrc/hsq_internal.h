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
constexpr int kMaxUSlicesSkinny = 16;  // U slices the skinny contraction prefetches
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
// The skinny contraction streams this part (half a byte per code).
//
// Layout version 2 appends the same codes as int8 operand bytes 16*code
// (the tiled contraction's B operand, moved global -> LDS unchanged): NT x
// Gp blocks of 1024 bytes, column-tile-major; block (nt, g) holds 64 lane
// slots of 16 bytes, slot l = output column 16*nt + l%16, channels
// 64g + 16*(l/16) + p at byte p.  Pad columns and the pad group hold 0.
// ---------------------------------------------------------------------------
inline int padded_groups(int K) { return ceil_div(K / kGroup, 2) * 2; }
// Scale groups of `group` channels (64 or 128): one scale per (row or
// column, group).  A group-128 scale covers two 64-channel blocks, which is
// one block pair of the packed residual.  The activation scales are stored
// per row tile for every padded 64-block (group 64) or every group (128).
inline int scale_groups_stored(int K, int group) { return group == kGroup ? padded_groups(K) : K / group; }
// nibble part (offset 0), int8 operand part (offset nibble_bytes), whole blob
inline size_t nibble_bytes(int K, int N) {
  return (size_t)ceil_div(N, kTile) * (size_t)(padded_groups(K) / 2) * 1024u;
}
inline size_t operand_bytes(int K, int N) { return (size_t)ceil_div(N, kTile) * (size_t)padded_groups(K) * 1024u; }
inline size_t packed_bytes(int K, int N) { return nibble_bytes(K, N) + operand_bytes(K, N); }

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
//   swp : batch x SWR x Npad float2, the weight scales as the tiled
//         contraction applies them, (sw/16, -1.5*2^23*sw/16) per (scale
//         group, column), written by its pre-pass; rows SG_w .. SWR-1, pad
//         columns and pad groups are zero (SWR = sw_pair_rows, Npad = N
//         rounded up to 16)
// ---------------------------------------------------------------------------
struct WsLayout {
  int MT = 0, G = 0, Gp = 0, Mpad = 0;
  int group = kGroup, bpg = 1, SG = 0;  // G = K/group scale groups; bpg = group/64 blocks each
  int u_slices = 0;      // S_u: K-slices of the quantization pass
  int swr = 0, npad = 0; // weight-scale pair rows and columns
  size_t qa_off = 0, sxs_off = 0, uw_off = 0, part_off = 0, swp_off = 0, total = 0;
};

// Rows of the weight-scale pair array: the scale groups of the stages (a
// stage is a 128-channel block pair: two groups of 64 or one of 128, the
// 64-channel groups padded to even), then one stage of zero rows that the
// stages past a workgroup's range read.
inline int sw_pair_rows(int K, int group) {
  return group == kGroup ? padded_groups(K) + 2 : K / group + 1;
}

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
  int asym;                // 1: asymmetric codes (q - z, zero point z per group)
  // public outputs (packed codes, fp16 scales, U as M x r)
  uint8_t *qx;
  uint16_t *sx;
  float *u_pub;
  // internal outputs (tiled codes, fp32 scales / 16, U slices)
  int8_t *qa;
  uint16_t *sxs;
  float *uw;
  int Gp, Mpad, ucols;
  // optional: the tiled contraction's weight-scale pairs, written by extra
  // workgroups of the first pass (swp == nullptr: none); sw is batch x swG x
  // swN fp16, the table batch x swr x swnpad pairs (sw_pair_item)
  const uint16_t *sw;
  float4 *swp;
  int swG, swN, swr, swnpad;
};

struct GemmArgs {
  const int8_t *qa;
  const uint16_t *sxs;
  const uint8_t *w;        // packed residual blob of projection 0 (nibble part first)
  size_t w_stride;         // bytes between projections' blobs
  size_t w_ops;            // offset of the int8 operand part within a blob
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
  // weight-scale pairs of the tiled contraction (see WsLayout)
  const float2 *swp;
  int swr, npad;
  // fused chain (tiled contraction, CHAIN mode): instead of Y, the epilogue
  // writes the next layer's input: act(Y) smoothed by lam2 and quantized
  // into that layer's workspace (codes qa2, scales sxs2), and the partial
  // sums of its rank-r2 down projection per 128-column block (upart2:
  // [column block][r2][Mpad]); optionally Y itself before the activation
  // (yhid, M x N fp32, a test export)
  int act;
  const uint16_t *lam2;
  const uint16_t *L1n;
  int r2, Gp2;
  int8_t *qa2;
  uint16_t *sxs2;
  float *upart2;
  float *yhid;
};

constexpr int kActIdentity = 0, kActGeluTanh = 1;
constexpr int kChainMaxRank = 8;   // rank of the next layer in a fused chain

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
// The tiled contraction's pre-pass: sw (batch x G x N fp16) -> the pair
// array a.swp (batch x a.swr x a.npad float2, layout in WsLayout).
hipError_t launch_sw_pairs(const GemmArgs &a, int batch, hipStream_t s);
// Split-K factor of the tiled contraction for this shape (1: no split) and
// the workspace bytes of its partial tiles.
int tiled_splits(int M, int N, int K, int r, int batch, int group);
size_t tiled_partial_bytes(int M, int N, int K, int r, int batch, int group);
hipError_t launch_gemm_skinny(const GemmArgs &a, int batch, bool dump, hipStream_t s);
// The tiled contraction with the CHAIN epilogue (one projection, unsplit,
// 8-wave workgroups), and the sum of its U partials into the next layer's
// single U slice: uw[j][m] = sum over column blocks of upart[blk][j][m].
hipError_t launch_gemm_tiled_chain(const GemmArgs &a, hipStream_t s);
hipError_t launch_chain_ureduce(const float *upart, int nblk, int r2, int Mpad, float *uw, hipStream_t s);

// block index -> (m-block, n-block).  Consecutive workgroup ids go to
// different XCDs (id % 8); regroup them so that XCD x owns a contiguous
// range of the tile order, and walk that order in groups of group_m
// m-blocks so concurrently running tiles share rows of A and columns of B.
__device__ __forceinline__ void xcd_tile_of(int bid, int nblk, int mblk, int group_m, int &mb, int &nb) {
  const int T = nblk * mblk;
  const int per = T / 8, rem = T % 8;
  const int x = bid % 8, loc = bid / 8;
  // XCD x owns [start(x), start(x) + per + (x < rem)); ids with loc == per
  // exist only for x < rem.
  const int t = x * per + min(x, rem) + loc;
  const int span = group_m * nblk;
  const int grp = t / span, first = grp * group_m;
  const int gsz = min(mblk - first, group_m);
  const int w = t % span;
  mb = first + w % gsz;
  nb = w / gsz;
}

// ---------------------------------------------------------------------------
// MX-fp4 variant (mx.hip)
// ---------------------------------------------------------------------------
struct MxLayout {
  int KS = 0, KS4 = 0, Mpad = 0;   // k-steps of 128 channels, groups of four k-steps, padded rows
  size_t qa_off = 0, sa_off = 0, u_off = 0, total = 0;
};

struct MxArgs {
  const uint16_t *X, *lam, *L1, *L2, *bias;
  uint8_t *qa, *sa;        // workspace: activation codes and scales (blob layout)
  float *U;                // workspace: r x Mpad
  const uint8_t *wq, *ws;  // packed weights: codes, scales
  void *Y;
  int y_bf16;
  int M, K, N, r, KS, KS4, Mpad;
  int u_slices;            // U partials, one per four k-steps (= KS4)
};

size_t mx_packed_bytes(int K, int N);
MxLayout plan_mx(int M, int K, int r);
hipError_t launch_mx_pack(const float *R, int K, int N, uint8_t *packed, hipStream_t s);
hipError_t launch_mx_linear(const MxArgs &a, hipStream_t s);

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

// Weight-scale pairs of the tiled contraction: item i covers 8 adjacent
// columns of one (projection, pair row) of the batch x swr x npad table and
// writes (sw/16, -1.5*2^23*sw/16) for each, zero past column N and past scale
// group G (the pad group and the zero stage); four 16-byte stores.
__device__ __forceinline__ void sw_pair_item(const uint16_t *__restrict__ sw, int G, int N, int swr, int npad,
                                             size_t i, float4 *__restrict__ out) {
  const int n0 = (int)(i % (npad / 8)) * 8;
  const size_t bg = i / (npad / 8);
  const int g = (int)(bg % swr), b = (int)(bg / swr);
  const uint16_t *row = sw + ((size_t)b * G + g) * N;
  float v[8];
  if ((N & 7) == 0 && g < G && n0 < N) {
    // whole 16-byte run (rows start 16-byte aligned when N % 8 == 0)
    const uint4 w = *reinterpret_cast<const uint4 *>(row + n0);
    const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f16_to_f32((uint16_t)(h[e / 2] >> (16 * (e & 1))));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n = n0 + e;
      v[e] = (g < G && n < N) ? f16_to_f32(row[n]) : 0.0f;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; e += 2)
    out[i * 4 + e / 2] = make_float4(v[e] * 0.0625f, -kMagic * 0.0625f * v[e], v[e + 1] * 0.0625f,
                                     -kMagic * 0.0625f * v[e + 1]);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Reductions over a row of 16 lanes through DPP (no LDS traffic): the
// butterfly quad-xor-1, quad-xor-2, half-row mirror, row mirror leaves the
// row's maximum / sum in every lane of the row, and since each step adds a
// value to its partner's in both orders, every lane holds the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));   // row_half_mirror
  return fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  return v + dpp_f32<0x140>(v);
}

// The activation quantizer's two roundings (the same arithmetic as the
// quantization pass): the fp16 scale of a group from its absmax (0 for a
// zero group, saturating at 65504), and a code clamp(rint(fl32(xh / s)),
// -8, 7) as the bits of 1.5 * 2^23 + code.
__device__ __forceinline__ uint16_t act_scale16(float amax) {
  if (amax == 0.0f) return 0;
  uint16_t s16 = f32_to_f16(amax / 7.0f);
  return s16 == 0x7C00u ? (uint16_t)0x7BFFu : s16;
}
__device__ __forceinline__ int act_code_bits(float xh, float inv_s) {
  const int v = __float_as_int(xh * inv_s + kMagic);
  return min(max(v, kMagicBits - 8), kMagicBits + 7);
}

// exp(x) in fp32 from basic operations only (each rounded once, no fused
// multiply-add), so that a plain fp32 implementation reproduces it bit for
// bit: x clamped to [-87, 88]; n = rint(x log2 e); Cody-Waite reduction
// r = x - n ln2 (ln2 split into 0.693145751953125 + 1.428606765330187e-6);
// the degree-6 Taylor polynomial of e^r in Horner form; times 2^n built
// from its exponent bits.  Relative error below 2^-21 on the range.
__device__ __forceinline__ float exp_f32_basic(float x) {
  x = fminf(fmaxf(x, -87.0f), 88.0f);
  const float n = __builtin_rintf(x * 1.44269504f);
  const float r = (x - n * 0.693145751953125f) - n * 1.428606765330187e-06f;
  float p = 1.388888888888889e-03f;              // 1/720
  p = p * r + 8.333333333333333e-03f;            // 1/120
  p = p * r + 4.166666666666666e-02f;            // 1/24
  p = p * r + 1.666666666666667e-01f;            // 1/6
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return p * __int_as_float(((int)n + 127) << 23);
}

// GELU in its tanh form, 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))),
// evaluated as y / (1 + exp(-2z)) with z = sqrt(2/pi) (y + 0.044715 y^3).
__device__ __forceinline__ float gelu_tanh_f32(float y) {
  const float y3 = (y * y) * y;
  const float z = 0.7978845608f * (y + 0.044715f * y3);
  return y / (1.0f + exp_f32_basic(-2.0f * z));
}

// Direct-to-LDS staging, shared by the tiled int4 and the MX contraction.
//
// End of a stage: this wave's loads (the next stage's direct-to-LDS blocks
// and its scale loads, all issued this stage) and its LDS reads and writes
// are complete, then the workgroup barrier.  After it every wave sees the
// next stage's operands in LDS, and no wave still reads the buffer the
// following stage's loads will overwrite.  (__syncthreads would add a
// release fence, which waits the same way but also stops the compiler from
// keeping loads in flight across it; here nothing is in flight.)
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct-to-LDS load of one 1 KB operand block (buffer_load_dwordx4 ...
// lds): lane l's 16 bytes, at voffset + soffset of the buffer resource rs
// (four dwords: base, stride, size, flags), land at LDS byte address
// lds + 16 l.  Written as an instruction of its own so that the compiler
// neither waits for it (the loads of stage s+1 stay in flight while stage s
// reads the other buffer) nor moves LDS accesses across it; stage_barrier
// is the wait.  It has no register results.
__device__ __forceinline__ void block_to_lds(v4u rs, uint32_t lds, uint32_t voffset, uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(rs), "s"(soffset)
               : "memory", "m0");
}

// The same for one dword per lane (256 bytes per wave): lane l's 4 bytes
// land at lds + 4 l.
__device__ __forceinline__ void dword_to_lds(v4u rs, uint32_t lds, uint32_t voffset, uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(rs), "s"(soffset)
               : "memory", "m0");
}

// A raw buffer resource as four scalar dwords (the layout the buffer
// instructions read): 48-bit base, stride 0, size in bytes (reads past it
// return zero), the same flags as buffer_rsrc.
__device__ __forceinline__ v4u raw_rsrc(const void *p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return (v4u){(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

// LDS byte address of a __shared__ object (for m0).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p);
}

}  // namespace hsq
#endif

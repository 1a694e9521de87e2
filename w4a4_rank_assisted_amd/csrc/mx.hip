// mx.hip -- the MX-fp4 format variant of the layer on gfx950's scaled MFMA.
//
// Same layer as the int4 path (W ~ L1 L2 + Q(R), smoothing by lambda, the
// rank-r branch on the smoothed activations: Deflating the Hessian,
// abstract), with both 4-bit operands in MX-fp4 (OCP Microscaling v1.0):
// per 32 consecutive values along K an e8m0 scale 2^X, X = floor(log2 amax)
// - 2 (byte X + 127, clamped to [0, 254]; 127 for a zero block), and e2m1
// elements rounded to nearest even, saturating at 6.
//
// One v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 operands covers a 16 x 16
// output tile and 128 channels (four 32-blocks).  Operand layout (measured):
// lane l holds row (A) or column (B) l % 16 and the 32 elements of block
// l / 16 of the 128, element 2i in the low nibble of byte i; the lane's e8m0
// byte scales exactly its own 32 elements.  The MFMA applies both scales and
// accumulates in fp32, so the main loop has no per-group rescale at all,
// unlike the int4 path.
//
// Blobs (KS = ceil(K / 128) k-steps, KS4 = ceil(KS / 4)):
//   operand blocks  [tile][KS][64 lanes][16 bytes]   (tile = 16 rows or columns)
//   scales          [tile][KS4][64 lanes][4 bytes]   (byte j: k-step 4 * ks4 + j)
// The packed weights are the W blob followed by its scales; the workspace
// holds 1/lambda, the activation blob, its scales and U.
#include "hsq_internal.h"

namespace hsq {

namespace {


typedef int v8i __attribute__((ext_vector_type(8)));

// e8m0 byte of a block's absmax: floor(log2 amax) is the fp32 exponent
// field minus 127 for a normal amax; a subnormal amax gives byte 0 (clamp)
__device__ __forceinline__ int mx_scale_byte(float amax) {
  if (amax == 0.0f) return 127;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return e - 2 < 0 ? 0 : e - 2;
}

// 32 values -> 16 bytes of codes (four dwords) and the scale byte.  v =
// x * 2^-X is exact (a power-of-two product whose result stays below 8); the
// packed fp4 down-conversion of gfx950 (divisor 1) rounds v to the nearest
// e2m1 value, ties to the even mantissa, saturates at 6 and keeps the sign
// bit; the first value of each pair goes to the low nibble of the byte
// selected by the last operand.
__device__ __forceinline__ int mx_block(const float (&x)[32], v4u &packed) {
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
  const int sb = mx_scale_byte(amax);
  const float inv = __int_as_float((254 - sb) << 23);   // 2^-(sb - 127), normal for sb in [0, 253]
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[8 * w + 0] * inv, x[8 * w + 1] * inv, 1.0f, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[8 * w + 2] * inv, x[8 * w + 3] * inv, 1.0f, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[8 * w + 4] * inv, x[8 * w + 5] * inv, 1.0f, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[8 * w + 6] * inv, x[8 * w + 7] * inv, 1.0f, 3);
    packed[w] = d;
  }
  return sb;
}

__global__ void k_mx_pack_w(const float *R, int K, int N, int KS, uint8_t *blob, uint8_t *scales) {
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  const int b = blockIdx.y * 4 + (threadIdx.x >> 6);    // 32-block along K
  if (n >= N || b >= 4 * KS) return;
  float x[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int k = 32 * b + e;
    x[e] = k < K ? R[(size_t)k * N + n] : 0.0f;
  }
  v4u p;
  const int sb = mx_block(x, p);
  const int nt = n >> 4, ks = b >> 2, lane = (n & 15) + 16 * (b & 3);
  *reinterpret_cast<v4u *>(blob + (((size_t)nt * KS + ks) * 64 + lane) * 16) = p;
  const int KS4 = (KS + 3) / 4;
  scales[(((size_t)nt * KS4 + (ks >> 2)) * 64 + lane) * 4 + (ks & 3)] = (uint8_t)sb;
}

// Activations: a workgroup takes one 16-row tile and 16 consecutive 32-blocks
// (four k-steps); thread t takes row t % 16 and block t / 16.  Its share of
// U is summed over the 16 threads of its row in block order through LDS and
// written as this slice's U partial (the contraction sums the slices in
// order).
template <int RP>
__global__ __launch_bounds__(256) void k_mx_quant(MxArgs a) {
  constexpr bool STAGE = RP > 0 && RP <= 8;      // L1 rows of the slice in LDS
  // one 32-channel block's L1 rows per LBS floats, padded by four so that
  // the blocks a wave reads at once sit in different banks
  constexpr int LBS = 32 * (RP > 0 ? RP : 1) + 4;
  __shared__ float us[16][16][RP > 0 ? RP : 1];
  __shared__ alignas(16) float l1s[STAGE ? 16 * LBS : 1];
  __shared__ alignas(16) float ils[512];           // fl32(1 / lambda) of the slice's channels
  const int tid = threadIdx.x, row = tid & 15, q = tid >> 4;
  const int mt = blockIdx.x, m = mt * 16 + row;
  const int nb = 4 * a.KS;                        // 32-blocks incl. the pad of the last k-step
  float u[RP > 0 ? RP : 1];
#pragma unroll
  for (int c = 0; c < (RP > 0 ? RP : 1); ++c) u[c] = 0.0f;
  const int k0 = 512 * blockIdx.y;
  for (int p = tid; p < 512; p += 256) ils[p] = k0 + p < a.K ? 1.0f / f16_to_f32(a.lam[k0 + p]) : 0.0f;
  if constexpr (STAGE) {
    for (int p = tid; p < 512 * RP; p += 256) {
      const int kk = p / RP, c = p % RP, k = k0 + kk;
      l1s[(kk >> 5) * LBS + (kk & 31) * RP + c] = (c < a.r && k < a.K) ? bf16_to_f32(a.L1[(size_t)k * a.r + c]) : 0.0f;
    }
  }
  __syncthreads();
  // this workgroup's slice: 16 blocks (one k-step group), one per thread row
  for (int b = 16 * blockIdx.y + q; b < min(nb, 16 * blockIdx.y + 16); b += 16) {
    float x[32];
    const bool live = m < a.M && 32 * b < a.K;
    if (live) {
      const v4u *src = reinterpret_cast<const v4u *>(a.X + (size_t)m * a.K + 32 * b);
      const v4f *il = reinterpret_cast<const v4f *>(ils + 32 * (b - 16 * (int)blockIdx.y));
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const v4u v = src[w];
        const v4f l0 = il[2 * w], l1 = il[2 * w + 1];
        x[8 * w + 0] = bf16_to_f32(v.x & 0xFFFFu) * l0.x;
        x[8 * w + 1] = bf16_to_f32(v.x >> 16) * l0.y;
        x[8 * w + 2] = bf16_to_f32(v.y & 0xFFFFu) * l0.z;
        x[8 * w + 3] = bf16_to_f32(v.y >> 16) * l0.w;
        x[8 * w + 4] = bf16_to_f32(v.z & 0xFFFFu) * l1.x;
        x[8 * w + 5] = bf16_to_f32(v.z >> 16) * l1.y;
        x[8 * w + 6] = bf16_to_f32(v.w & 0xFFFFu) * l1.z;
        x[8 * w + 7] = bf16_to_f32(v.w >> 16) * l1.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = 0.0f;
    }
    v4u p;
    const int sb = mx_block(x, p);
    const int ks = b >> 2, lane = row + 16 * (b & 3);
    *reinterpret_cast<v4u *>(a.qa + (((size_t)mt * a.KS + ks) * 64 + lane) * 16) = p;
    a.sa[(((size_t)mt * a.KS4 + (ks >> 2)) * 64 + lane) * 4 + (ks & 3)] = (uint8_t)sb;
    if constexpr (STAGE) {
      if (live) {
        const float *lr = l1s + (b - 16 * (int)blockIdx.y) * LBS;
#pragma unroll
        for (int e = 0; e < 32; ++e)
#pragma unroll
          for (int c = 0; c < RP; ++c) u[c] = __builtin_fmaf(x[e], lr[e * RP + c], u[c]);
      }
    } else if constexpr (RP > 0) {
      if (live && (a.r & 3) == 0) {
        // four rank columns per 8-byte load
#pragma unroll 4
        for (int e = 0; e < 32; ++e) {
          const v2u *l1 = reinterpret_cast<const v2u *>(a.L1 + (size_t)(32 * b + e) * a.r);
#pragma unroll
          for (int c4 = 0; c4 < RP / 4; ++c4) {
            if (4 * c4 >= a.r) break;
            const v2u w = l1[c4];
            u[4 * c4 + 0] = __builtin_fmaf(x[e], bf16_to_f32(w.x & 0xFFFFu), u[4 * c4 + 0]);
            u[4 * c4 + 1] = __builtin_fmaf(x[e], bf16_to_f32(w.x >> 16), u[4 * c4 + 1]);
            u[4 * c4 + 2] = __builtin_fmaf(x[e], bf16_to_f32(w.y & 0xFFFFu), u[4 * c4 + 2]);
            u[4 * c4 + 3] = __builtin_fmaf(x[e], bf16_to_f32(w.y >> 16), u[4 * c4 + 3]);
          }
        }
      } else if (live) {
#pragma unroll 4
        for (int e = 0; e < 32; ++e) {
          const uint16_t *l1 = a.L1 + (size_t)(32 * b + e) * a.r;
#pragma unroll
          for (int c = 0; c < RP; ++c)
            if (c < a.r) u[c] = __builtin_fmaf(x[e], bf16_to_f32(l1[c]), u[c]);
        }
      }
    }
  }
  if constexpr (RP > 0) {
#pragma unroll
    for (int c = 0; c < RP; ++c) us[row][q][c] = u[c];
    __syncthreads();
    for (int it = tid; it < 16 * RP; it += 256) {
      const int rr = it & 15, c = it >> 4;
      float s = 0.0f;
      for (int j = 0; j < 16; ++j) s += us[rr][j][c];
      if (c < a.r) a.U[((size_t)blockIdx.y * a.r + c) * a.Mpad + mt * 16 + rr] = s;
    }
  }
}

template <int V>
struct int_c {
  static constexpr int value = V;
};

// The residual contraction with the epilogue.  A workgroup of WGM x WGN
// waves owns (TMW * WGM) x (TNW * WGN) MFMA tiles; each wave TMW x TNW of
// them.  One k-step (128 channels) per stage; the operand blocks go
// global -> registers -> LDS with the loads of stage s + 2 issued at the
// start of stage s into one of two register slots (slot = stage parity,
// fixed at compile time by unrolling), two LDS buffers, one barrier per
// stage.  The e8m0 scales (one dword per tile and lane for four k-steps,
// byte j picked by a shift) ride the same pipeline: a group of four
// k-steps needs (AT + BT) x 64 dwords, loaded a quarter per stage with the
// operands of the group before and written into one of two LDS scale
// buffers, so that the first stage of a group reads its scales from LDS
// instead of waiting on memory.  Workgroups walk the tiles in the
// XCD-grouped order of xcd_tile_of.
template <int TMW, int TNW, int WGM, int WGN, int RPT, int GROUPM = 8>
__global__ __launch_bounds__(64 * WGM * WGN, 2) void k_mx_gemm(MxArgs a) {
  constexpr int NTHR = 64 * WGM * WGN;
  constexpr int AT = TMW * WGM, BT = TNW * WGN;          // tiles of the workgroup
  constexpr int LA = AT * 64 / NTHR, LB = BT * 64 / NTHR; // 16-byte slots per thread and stage
  static_assert(AT * 64 % NTHR == 0 && BT * 64 % NTHR == 0, "whole slots per thread");
  constexpr int BMR = AT * 16, BNC = BT * 16;            // rows, columns of the workgroup
  __shared__ alignas(16) uint8_t opa[2][AT][64][16];
  __shared__ alignas(16) uint8_t opb[2][BT][64][16];
  constexpr int SCW = (AT + BT) * 64;                     // scale dwords of a group of four k-steps
  constexpr int SQ = SCW / 4;                             // scale dwords per stage: a quarter of a group's
  static_assert(AT == BT && SQ % 64 == 0 && SQ <= NTHR, "quarters 0, 1: A tiles; 2, 3: B tiles; one dword per thread");
  __shared__ uint32_t ssc[2][SCW];                        // [group parity][A tiles, then B tiles][lane]
  __shared__ float eu[RPT > 0 ? RPT : 1][BMR];
  __shared__ float el2[RPT > 0 ? RPT : 1][BNC];
  __shared__ float ebias[BNC];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int nblk = (a.N + BNC - 1) / BNC, mblk = (a.Mpad / 16 + AT - 1) / AT;
  int mb, nb;
  xcd_tile_of(blockIdx.x, nblk, mblk, GROUPM, mb, nb);
  const int mt0 = mb * AT, nt0 = nb * BT;
  const int MT = a.Mpad / 16, NT = (a.N + 15) / 16;
  const int KS = a.KS, KS4 = a.KS4;
  // buffer loads: one per-lane offset, the tile and k-step in a scalar
  // offset (the tile a thread loads depends on its wave only)
  const __amdgpu_buffer_rsrc_t rs_qa = buffer_rsrc(a.qa, (uint32_t)MT * KS * 1024);
  const __amdgpu_buffer_rsrc_t rs_wq = buffer_rsrc(a.wq, (uint32_t)NT * KS * 1024);
  const __amdgpu_buffer_rsrc_t rs_sa = buffer_rsrc(a.sa, (uint32_t)MT * KS4 * 256);
  const __amdgpu_buffer_rsrc_t rs_sb = buffer_rsrc(a.ws, (uint32_t)NT * KS4 * 256);
  const uint32_t vo16 = (uint32_t)lane * 16, vo4 = (uint32_t)lane * 4;

  v4f acc[TMW][TNW];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // the scale dword of quarter P of a group: A tiles (P = 0, 1: tiles 4P ..
  // 4P + 3) or B tiles (P = 2, 3), one lane slot per thread
  auto scale_word = [&](int g, auto pc) __attribute__((always_inline)) -> uint32_t {
    constexpr int P = decltype(pc)::value;
    const int tile = (P & 1) * (SQ / 64) + wave;      // (threads tid < SQ, waves wave < SQ / 64)
    if constexpr (P < 2)
      return __builtin_amdgcn_raw_buffer_load_b32(rs_sa, vo4, (min(mt0 + tile, MT - 1) * KS4 + g) * 256, 0);
    else
      return __builtin_amdgcn_raw_buffer_load_b32(rs_sb, vo4, (min(nt0 + tile, NT - 1) * KS4 + g) * 256, 0);
  };
  v4u ra[2][LA], rb[2][LB];
  uint32_t rs[2];
  // operands of k-step ks and quarter P = ks % 4 of the next group's scales
  auto load = [&](int ks, auto sc, auto pc) __attribute__((always_inline)) {
    constexpr int SL = decltype(sc)::value;
    const int k = min(ks, KS - 1);                   // past the end: a clamped, unused reload
#pragma unroll
    for (int u = 0; u < LA; ++u)
      ra[SL][u] = __builtin_amdgcn_raw_buffer_load_b128(rs_qa, vo16, (min(mt0 + wave + u * (NTHR / 64), MT - 1) * KS + k) * 1024, 0);
#pragma unroll
    for (int u = 0; u < LB; ++u)
      rb[SL][u] = __builtin_amdgcn_raw_buffer_load_b128(rs_wq, vo16, (min(nt0 + wave + u * (NTHR / 64), NT - 1) * KS + k) * 1024, 0);
    if (SQ == NTHR || tid < SQ) rs[SL] = scale_word(min(ks / 4 + 1, KS4 - 1), pc);
  };
  auto store = [&](int buf, int ks, auto sc, auto pc) __attribute__((always_inline)) {
    constexpr int SL = decltype(sc)::value;
    constexpr int P = decltype(pc)::value;
#pragma unroll
    for (int u = 0; u < LA; ++u)
      *reinterpret_cast<v4u *>(&opa[buf][(tid >> 6) + u * (NTHR / 64)][lane][0]) = ra[SL][u];
#pragma unroll
    for (int u = 0; u < LB; ++u)
      *reinterpret_cast<v4u *>(&opb[buf][(tid >> 6) + u * (NTHR / 64)][lane][0]) = rb[SL][u];
    if (SQ == NTHR || tid < SQ) ssc[(ks / 4 + 1) & 1][P * SQ + tid] = rs[SL];
  };

  // prologue: group 0's scales, the first two k-steps' operands and the
  // epilogue operands all in flight together, so the first stores wait on
  // one memory round trip
  uint32_t s0[4] = {0u, 0u, 0u, 0u};
  if (SQ == NTHR || tid < SQ) {
    s0[0] = scale_word(0, int_c<0>{});
    s0[1] = scale_word(0, int_c<1>{});
    s0[2] = scale_word(0, int_c<2>{});
    s0[3] = scale_word(0, int_c<3>{});
  }
  load(0, int_c<0>{}, int_c<0>{});
  load(1, int_c<1>{}, int_c<1>{});
  // epilogue operands: U (its K-slices summed in order; the first
  // kMaxUSlices loaded together, clamped addresses), L2, bias
  for (int p = tid; p < RPT * BMR; p += NTHR) {
    const int c = p / BMR, rr = p % BMR, m = mt0 * 16 + rr;
    const int cc = min(c, a.r - 1), mm = min(m, a.Mpad - 1);
    float us[kMaxUSlices];
#pragma unroll
    for (int sl = 0; sl < kMaxUSlices; ++sl)
      us[sl] = a.U[((size_t)min(sl, a.u_slices - 1) * a.r + cc) * a.Mpad + mm];
    float u = 0.0f;
#pragma unroll
    for (int sl = 0; sl < kMaxUSlices; ++sl)
      if (sl < a.u_slices) u += us[sl];
    for (int sl = kMaxUSlices; sl < a.u_slices; ++sl) u += a.U[((size_t)sl * a.r + cc) * a.Mpad + mm];
    eu[c][rr] = (c < a.r && m < a.M) ? u : 0.0f;
  }
  for (int p = tid; p < RPT * BNC; p += NTHR) {
    const int c = p / BNC, cc = p % BNC, n = nt0 * 16 + cc;
    el2[c][cc] = (c < a.r && n < a.N) ? bf16_to_f32(a.L2[(size_t)c * a.N + n]) : 0.0f;
  }
  for (int p = tid; p < BNC; p += NTHR) {
    const int n = nt0 * 16 + p;
    ebias[p] = (a.bias && n < a.N) ? bf16_to_f32(a.bias[n]) : 0.0f;
  }
  if (SQ == NTHR || tid < SQ) {
    ssc[0][tid] = s0[0];
    ssc[0][SQ + tid] = s0[1];
    ssc[0][2 * SQ + tid] = s0[2];
    ssc[0][3 * SQ + tid] = s0[3];
  }
  store(0, 0, int_c<0>{}, int_c<0>{});
  __syncthreads();

  uint32_t scA[TMW], scB[TNW];
  // stage ks: J = ks % 4 (scale byte), slot and buffer = ks % 2
  auto stage = [&](int ks, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    constexpr int SL = J & 1;
    if (J == 0) {
      const uint32_t *sc = ssc[(ks >> 2) & 1];
#pragma unroll
      for (int i = 0; i < TMW; ++i) scA[i] = sc[(wm * TMW + i) * 64 + lane];
#pragma unroll
      for (int j = 0; j < TNW; ++j) scB[j] = sc[AT * 64 + (wn * TNW + j) * 64 + lane];
    }
    load(ks + 2, int_c<SL>{}, int_c<(J + 2) & 3>{});  // this slot's data went to LDS a stage ago
    v8i bv[TNW];
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const v4u v = *reinterpret_cast<const v4u *>(&opb[SL][wn * TNW + j][lane][0]);
      bv[j] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
      const v4u v = *reinterpret_cast<const v4u *>(&opa[SL][wm * TMW + i][lane][0]);
      const v8i av = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      const int sa_b = (int)((scA[i] >> (8 * J)) & 0xFFu);
#pragma unroll
      for (int j = 0; j < TNW; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv[j], acc[i][j], 4, 4, 0, sa_b, 0,
                                                                     (int)((scB[j] >> (8 * J)) & 0xFFu));
    }
    if (ks + 1 < KS) store(SL ^ 1, ks + 1, int_c<SL ^ 1>{}, int_c<(J + 1) & 3>{});
    __syncthreads();
  };
  int ks = 0;
  for (; ks + 4 <= KS; ks += 4) {
    stage(ks, int_c<0>{});
    stage(ks + 1, int_c<1>{});
    stage(ks + 2, int_c<2>{});
    stage(ks + 3, int_c<3>{});
  }
  if (ks < KS) stage(ks, int_c<0>{});
  if (ks + 1 < KS) stage(ks + 1, int_c<1>{});
  if (ks + 2 < KS) stage(ks + 2, int_c<2>{});

  // epilogue: Y = acc + U L2 + bias; per row tile the wave's 16 x WCOL
  // values go through a wave-private LDS region (the operand buffers are
  // free after the last barrier) and leave as 16-byte row-contiguous stores
  constexpr int WCOL = TNW * 16;
  static_assert(WGM * WGN * 16 * WCOL * 4 <= (int)sizeof(opa), "transpose region");
  char *tb = reinterpret_cast<char *>(&opa[0][0][0][0]) + wave * (16 * WCOL * 4);
  const int rowq = 4 * (lane >> 4), colq = lane & 15;
  const int yb = a.y_bf16 ? 2 : 4, per16 = 16 / yb, cpr = WCOL / per16;
  const bool vec_ok = (a.N % per16) == 0;
  const int ncol0 = (nt0 + wn * TNW) * 16;
#pragma unroll
  for (int i = 0; i < TMW; ++i) {
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const int cc = (wn * TNW + j) * 16 + colq;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int rr = (wm * TMW + i) * 16 + rowq + qq;
        float y = acc[i][j][qq];
#pragma unroll
        for (int c = 0; c < RPT; ++c) y = __builtin_fmaf(eu[c][rr], el2[c][cc], y);
        y += ebias[cc];
        const int off = (rowq + qq) * WCOL + j * 16 + colq;
        if (a.y_bf16)
          reinterpret_cast<uint16_t *>(tb)[off] = f32_to_bf16(y);
        else
          reinterpret_cast<float *>(tb)[off] = y;
      }
    }
    const int mrow0 = (mt0 + wm * TMW + i) * 16;
    for (int k = lane; k < 16 * cpr; k += 64) {
      const int row = k / cpr, ch = k % cpr;
      const int m = mrow0 + row, n = ncol0 + ch * per16;
      if (m >= a.M || n >= a.N) continue;
      const v4u v = *reinterpret_cast<const v4u *>(tb + (row * WCOL + ch * per16) * yb);
      char *dst = reinterpret_cast<char *>(a.Y) + ((size_t)m * a.N + n) * yb;
      if (vec_ok && n + per16 <= a.N) {
        *reinterpret_cast<v4u *>(dst) = v;
      } else if (a.y_bf16) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < a.N) reinterpret_cast<uint16_t *>(dst)[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) reinterpret_cast<uint32_t *>(dst)[e] = v[e];
      }
    }
  }
}

// workgroup 128 x 128: 2 x 4 waves of 64 x 32 (104 VGPRs, four waves per
// SIMD).  Measured against 2 x 2 waves of 64 x 64 (248 VGPRs, two waves
// per SIMD): 13 % faster at pixart size, 8 % on the FLUX and Qwen3 up
// layers; a 256 x 128 workgroup ran at one wave per SIMD and was slower.
template <int RP, int TMW>
hipError_t launch_mx_gemm(const MxArgs &a, hipStream_t s) {
  constexpr int TNW = 2, WGM = 2, WGN = 4;
  const int tiles = ceil_div(a.N, 16 * TNW * WGN) * ceil_div(a.M, 16 * TMW * WGM);
  hipLaunchKernelGGL((k_mx_gemm<TMW, TNW, WGM, WGN, RP>), dim3((unsigned)tiles), dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int RP>
hipError_t launch_mx_rp(const MxArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_mx_quant<RP>, dim3((unsigned)(a.Mpad / 16), (unsigned)a.u_slices), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mx_gemm<RP, 4>(a, s);
}

}  // namespace

size_t mx_packed_bytes(int K, int N) {
  const int KS = ceil_div(K, 128), KS4 = ceil_div(KS, 4), NT = ceil_div(N, 16);
  return (size_t)NT * KS * 1024 + (size_t)NT * KS4 * 256;
}

MxLayout plan_mx(int M, int K, int r) {
  MxLayout L;
  L.KS = ceil_div(K, 128);
  L.KS4 = ceil_div(L.KS, 4);
  L.Mpad = ceil_div(M, 16) * 16;
  size_t off = 0;
  L.qa_off = off;
  off = align_up(off + (size_t)(L.Mpad / 16) * L.KS * 1024, 256);
  L.sa_off = off;
  off = align_up(off + (size_t)(L.Mpad / 16) * L.KS4 * 256, 256);
  L.u_off = off;
  off = align_up(off + (size_t)L.KS4 * r * L.Mpad * sizeof(float), 256);
  L.total = off;
  return L;
}

hipError_t launch_mx_pack(const float *R, int K, int N, uint8_t *packed, hipStream_t s) {
  const int KS = ceil_div(K, 128), NT = ceil_div(N, 16);
  hipLaunchKernelGGL(k_mx_pack_w, dim3((unsigned)ceil_div(N, 64), (unsigned)KS), dim3(256), 0, s, R, K, N, KS,
                     packed, packed + (size_t)NT * KS * 1024);
  return hipGetLastError();
}

hipError_t launch_mx_linear(const MxArgs &a, hipStream_t s) {
  if (a.r == 0) return launch_mx_rp<0>(a, s);
  if (a.r <= 4) return launch_mx_rp<4>(a, s);
  if (a.r <= 8) return launch_mx_rp<8>(a, s);
  if (a.r <= 16) return launch_mx_rp<16>(a, s);
  return launch_mx_rp<32>(a, s);
}

}  // namespace hsq

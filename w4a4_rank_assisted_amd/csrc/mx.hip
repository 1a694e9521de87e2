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

#include <type_traits>

namespace hsq {

namespace {


typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kMxCUs = 256;   // compute units of the MI355X

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

// The residual contraction with the epilogue.  Workgroup 128 x 128 outputs:
// 2 x 4 waves, each 64 x 32 = 4 x 2 MFMA tiles.  A stage is two k-steps
// (256 channels): wave w moves A tile w and B tile w of both k-steps global
// -> LDS with direct-to-LDS loads (four 1 KB blocks, no register staging),
// into one of two stage buffers; the loads of stage t + 1 are issued as
// stage t starts, and one barrier ends each stage (the wait of
// stage_barrier covers the loads).  The e8m0 scales (one dword per tile and
// lane for a group of four k-steps, byte j = k-step 4g + j) move the same
// way, one group ahead, into one of two scale buffers; a wave reads its
// tiles' dwords at the first stage of each group.  An odd last k-step
// skips the second half of its stage.  Workgroups walk the tiles in the
// XCD-grouped order of xcd_tile_of.  The epilogue operands (U summed over
// its K-slices in order, L2, bias) are loaded with the first stage for rank
// up to 4, after the last one into the then free stage buffers otherwise
// (their arrays would not leave room for two workgroups per CU).
template <int RPT, int GROUPM = 8>
__global__ __launch_bounds__(512, 2) void k_mx_gemm(MxArgs a) {
  constexpr int TMW = 4, TNW = 2, WGM = 2, WGN = 4, NTHR = 64 * WGM * WGN;
  constexpr int AT = TMW * WGM, BT = TNW * WGN;           // tiles of the workgroup (one per wave)
  static_assert(AT == NTHR / 64 && BT == NTHR / 64, "wave w moves A tile w and B tile w");
  constexpr int BMR = AT * 16, BNC = BT * 16;             // rows, columns of the workgroup
  constexpr int KSS = 2;                                  // k-steps per stage
  struct Ops {
    uint8_t a[KSS][AT][64][16];
    uint8_t b[KSS][BT][64][16];
  };
  __shared__ alignas(16) Ops ops[2];
  __shared__ uint32_t ssc[2][(AT + BT) * 64];             // [group parity][A tiles, then B tiles][lane]
  constexpr bool EARLY = RPT <= 4;                        // epilogue operands with the first stage
  constexpr int RE = RPT > 0 ? RPT : 1;
  __shared__ float epi_early[EARLY ? 2 * RE * 128 + 128 : 1];
  static_assert(RE * BMR * 4 <= (int)sizeof(ops[1].a) && RE * BNC * 4 <= (int)sizeof(ops[1].b) &&
                BNC * 4 <= (int)sizeof(ops[0].b), "late epilogue operands fit the stage buffers");
  float *eu = EARLY ? epi_early : reinterpret_cast<float *>(&ops[1].a[0][0][0][0]);          // [RPT][BMR]
  float *el2 = EARLY ? epi_early + RE * BMR : reinterpret_cast<float *>(&ops[1].b[0][0][0][0]);  // [RPT][BNC]
  float *eb = EARLY ? epi_early + 2 * RE * 128 : reinterpret_cast<float *>(&ops[0].b[0][0][0][0]);  // [BNC]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int nblk = (a.N + BNC - 1) / BNC, mblk = (a.Mpad / 16 + AT - 1) / AT;
  int mb, nb;
  xcd_tile_of(blockIdx.x, nblk, mblk, GROUPM, mb, nb);
  const int mt0 = mb * AT, nt0 = nb * BT;
  const int MT = a.Mpad / 16, NT = (a.N + 15) / 16;
  const int KS = a.KS, KS4 = a.KS4, nst = (KS + 1) / 2;
  // tiles past the matrix reload the last one (their outputs are not stored)
  const int ta = min(mt0 + wave, MT - 1), tb = min(nt0 + wave, NT - 1);
  const v4u rq = raw_rsrc(a.qa, (uint32_t)MT * KS * 1024), rw = raw_rsrc(a.wq, (uint32_t)NT * KS * 1024);
  const v4u rsa = raw_rsrc(a.sa, (uint32_t)MT * KS4 * 256), rsb = raw_rsrc(a.ws, (uint32_t)NT * KS4 * 256);
  const uint32_t vo16 = (uint32_t)lane * 16, vo4 = (uint32_t)lane * 4;

  auto issue_stage = [&](int t, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KSS; ++kk) {
      const int k = min(KSS * t + kk, KS - 1);
      block_to_lds(rq, lds_addr(&ops[buf].a[kk][wave][0][0]), vo16, (uint32_t)(ta * KS + k) * 1024u);
      block_to_lds(rw, lds_addr(&ops[buf].b[kk][wave][0][0]), vo16, (uint32_t)(tb * KS + k) * 1024u);
    }
  };
  auto issue_scales = [&](int g) __attribute__((always_inline)) {
    uint32_t *dst = ssc[g & 1];
    dword_to_lds(rsa, lds_addr(dst + wave * 64), vo4, (uint32_t)(ta * KS4 + g) * 256u);
    dword_to_lds(rsb, lds_addr(dst + (AT + wave) * 64), vo4, (uint32_t)(tb * KS4 + g) * 256u);
  };
  auto load_epilogue = [&]() __attribute__((always_inline)) {
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
      eu[c * BMR + rr] = (c < a.r && m < a.M) ? u : 0.0f;
    }
    for (int p = tid; p < RPT * BNC; p += NTHR) {
      const int c = p / BNC, cc = p % BNC, n = nt0 * 16 + cc;
      el2[c * BNC + cc] = (c < a.r && n < a.N) ? bf16_to_f32(a.L2[(size_t)c * a.N + n]) : 0.0f;
    }
    for (int p = tid; p < BNC; p += NTHR) {
      const int n = nt0 * 16 + p;
      eb[p] = (a.bias && n < a.N) ? bf16_to_f32(a.bias[n]) : 0.0f;
    }
  };

  v4f acc[TMW][TNW];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  issue_scales(0);
  issue_stage(0, 0);
  if constexpr (EARLY) load_epilogue();
  stage_barrier();

  uint32_t scA[TMW], scB[TNW];
  for (int t = 0; t < nst; ++t) {
    const int buf = t & 1;
    if (t + 1 < nst) issue_stage(t + 1, buf ^ 1);
    if ((t & 1) == 0) {
      // first stage of group g: its scales arrived a stage ago (or in the
      // prologue); the next group's go to the other scale buffer, whose
      // last readers finished before the previous barrier
      const int g = t >> 1;
      const uint32_t *sc = ssc[g & 1];
#pragma unroll
      for (int i = 0; i < TMW; ++i) scA[i] = sc[(wm * TMW + i) * 64 + lane];
#pragma unroll
      for (int j = 0; j < TNW; ++j) scB[j] = sc[(AT + wn * TNW + j) * 64 + lane];
      if (g + 1 < KS4) issue_scales(g + 1);
    }
#pragma unroll
    for (int kk = 0; kk < KSS; ++kk) {
      if (kk > 0 && KSS * t + kk >= KS) break;          // odd last k-step (uniform)
      const int J = 2 * (t & 1) + kk;                    // scale byte of this k-step
      v8i bv[TNW];
#pragma unroll
      for (int j = 0; j < TNW; ++j) {
        const v4u v = *reinterpret_cast<const v4u *>(&ops[buf].b[kk][wn * TNW + j][lane][0]);
        bv[j] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < TMW; ++i) {
        const v4u v = *reinterpret_cast<const v4u *>(&ops[buf].a[kk][wm * TMW + i][lane][0]);
        const v8i av = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        const int sa_b = (int)((scA[i] >> (8 * J)) & 0xFFu);
#pragma unroll
        for (int j = 0; j < TNW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv[j], acc[i][j], 4, 4, 0, sa_b, 0,
                                                                       (int)((scB[j] >> (8 * J)) & 0xFFu));
      }
    }
    stage_barrier();
  }
  if constexpr (!EARLY) {
    load_epilogue();
    __syncthreads();
  }

  // epilogue: Y = acc + U L2 + bias; per row tile the wave's 16 x WCOL
  // values go through a wave-private LDS region of stage buffer 0's A part
  // and leave as 16-byte row-contiguous stores
  constexpr int WCOL = TNW * 16;
  static_assert(WGM * WGN * 16 * WCOL * 4 <= (int)sizeof(ops[0].a), "transpose region");
  char *tbuf = reinterpret_cast<char *>(&ops[0].a[0][0][0][0]) + wave * (16 * WCOL * 4);
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
        for (int c = 0; c < RPT; ++c) y = __builtin_fmaf(eu[c * BMR + rr], el2[c * BNC + cc], y);
        y += eb[cc];
        const int off = (rowq + qq) * WCOL + j * 16 + colq;
        if (a.y_bf16)
          reinterpret_cast<uint16_t *>(tbuf)[off] = f32_to_bf16(y);
        else
          reinterpret_cast<float *>(tbuf)[off] = y;
      }
    }
    const int mrow0 = (mt0 + wm * TMW + i) * 16;
    for (int k = lane; k < 16 * cpr; k += 64) {
      const int row = k / cpr, ch = k % cpr;
      const int m = mrow0 + row, n = ncol0 + ch * per16;
      if (m >= a.M || n >= a.N) continue;
      const v4u v = *reinterpret_cast<const v4u *>(tbuf + (row * WCOL + ch * per16) * yb);
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

// Wide wave tiles: workgroup 128 x 256 outputs, 2 x 4 waves of 64 x 64
// (4 x 4 MFMA tiles).  Per k-step a wave reads 4 A and 4 B operand blocks
// for 16 MFMAs: half an LDS read per MFMA, where 64 x 32 needs three
// quarters.  A stage is one k-step: wave w moves A tile w and B tiles w and
// w + 8 (three 1 KB direct-to-LDS loads) into one of two stage buffers; the
// e8m0 scales of a group of four k-steps (the same tiles) move one group
// ahead.  The four k-steps of a group are unrolled, so the MFMA takes its
// scale byte from the group's dword by its byte select (op_sel), with no
// extraction.  Epilogue operands load with the first stage.
template <int RPT, int GROUPM = 8>
__global__ __launch_bounds__(512, 4) void k_mx_gemm_w(MxArgs a) {
  constexpr int TMW = 4, TNW = 4, WGM = 2, WGN = 4, NTHR = 64 * WGM * WGN;
  constexpr int AT = TMW * WGM, BT = TNW * WGN;           // 8 A tiles, 16 B tiles
  static_assert(AT == NTHR / 64 && BT == 2 * AT, "wave w moves A tile w and B tiles w, w + AT");
  constexpr int BMR = AT * 16, BNC = BT * 16;             // 128 rows, 256 columns
  struct Ops {
    uint8_t a[AT][64][16];
    uint8_t b[BT][64][16];
  };
  __shared__ alignas(16) Ops ops[2];
  __shared__ uint32_t ssc[2][(AT + BT) * 64];             // [group parity][A tiles, then B tiles][lane]
  constexpr int RE = RPT > 0 ? RPT : 1;
  __shared__ float eu[RE * BMR], el2[RE * BNC], eb[BNC];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int nblk = (a.N + BNC - 1) / BNC, mblk = (a.Mpad / 16 + AT - 1) / AT;
  int mb, nb;
  xcd_tile_of(blockIdx.x, nblk, mblk, GROUPM, mb, nb);
  const int mt0 = mb * AT, nt0 = nb * BT;
  const int MT = a.Mpad / 16, NT = (a.N + 15) / 16;
  const int KS = a.KS, KS4 = a.KS4;
  // tiles past the matrix reload the last one (their outputs are not stored)
  const int ta = min(mt0 + wave, MT - 1);
  const int tb0 = min(nt0 + wave, NT - 1), tb1 = min(nt0 + AT + wave, NT - 1);
  const v4u rq = raw_rsrc(a.qa, (uint32_t)MT * KS * 1024), rw = raw_rsrc(a.wq, (uint32_t)NT * KS * 1024);
  const v4u rsa = raw_rsrc(a.sa, (uint32_t)MT * KS4 * 256), rsb = raw_rsrc(a.ws, (uint32_t)NT * KS4 * 256);
  const uint32_t vo16 = (uint32_t)lane * 16, vo4 = (uint32_t)lane * 4;

  auto issue_stage = [&](int k, int buf) __attribute__((always_inline)) {
    block_to_lds(rq, lds_addr(&ops[buf].a[wave][0][0]), vo16, (uint32_t)(ta * KS + k) * 1024u);
    block_to_lds(rw, lds_addr(&ops[buf].b[wave][0][0]), vo16, (uint32_t)(tb0 * KS + k) * 1024u);
    block_to_lds(rw, lds_addr(&ops[buf].b[AT + wave][0][0]), vo16, (uint32_t)(tb1 * KS + k) * 1024u);
  };
  auto issue_scales = [&](int g) __attribute__((always_inline)) {
    uint32_t *dst = ssc[g & 1];
    dword_to_lds(rsa, lds_addr(dst + wave * 64), vo4, (uint32_t)(ta * KS4 + g) * 256u);
    dword_to_lds(rsb, lds_addr(dst + (AT + wave) * 64), vo4, (uint32_t)(tb0 * KS4 + g) * 256u);
    dword_to_lds(rsb, lds_addr(dst + (2 * AT + wave) * 64), vo4, (uint32_t)(tb1 * KS4 + g) * 256u);
  };
  auto load_epilogue = [&]() __attribute__((always_inline)) {
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
      eu[c * BMR + rr] = (c < a.r && m < a.M) ? u : 0.0f;
    }
    for (int p = tid; p < RPT * BNC; p += NTHR) {
      const int c = p / BNC, cc = p % BNC, n = nt0 * 16 + cc;
      el2[c * BNC + cc] = (c < a.r && n < a.N) ? bf16_to_f32(a.L2[(size_t)c * a.N + n]) : 0.0f;
    }
    for (int p = tid; p < BNC; p += NTHR) {
      const int n = nt0 * 16 + p;
      eb[p] = (a.bias && n < a.N) ? bf16_to_f32(a.bias[n]) : 0.0f;
    }
  };

  v4f acc[TMW][TNW];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  issue_scales(0);
  issue_stage(0, 0);
  load_epilogue();
  stage_barrier();

  // one k-step: its operands are in stage buffer J & 1 (the group's first
  // k-step is even), its scales in byte J of the group's dwords
  auto kstep = [&](auto jc, const uint32_t (&scA)[TMW], const uint32_t (&scB)[TNW]) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value, BUF = J & 1;
    v8i bv[TNW];
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const v4u v = *reinterpret_cast<const v4u *>(&ops[BUF].b[wn * TNW + j][lane][0]);
      bv[j] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
      const v4u v = *reinterpret_cast<const v4u *>(&ops[BUF].a[wm * TMW + i][lane][0]);
      const v8i av = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < TNW; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv[j], acc[i][j], 4, 4, J, (int)scA[i], J,
                                                                     (int)scB[j]);
    }
    // the k-step's results pinned here: the next k-step's MFMAs cannot
    // move above its barrier (interleaved k-steps keep twice the
    // accumulators alive)
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
      for (int j = 0; j < TNW; ++j) asm volatile("" : "+v"(acc[i][j]));
  };
  // k-step t = 4 g + J: the next k-step's operands are issued first (into
  // the other buffer); one barrier ends the k-step
  auto step = [&](auto jc, int t, const uint32_t (&scA)[TMW], const uint32_t (&scB)[TNW])
      __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    if (t + 1 < KS) issue_stage(t + 1, (J & 1) ^ 1);
    kstep(jc, scA, scB);
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // the group's scales arrived before the last barrier; the next group's go
  // to the other scale buffer, whose last readers finished before the
  // barrier of the previous group's first k-step
  auto group_scales = [&](int g, uint32_t (&scA)[TMW], uint32_t (&scB)[TNW]) __attribute__((always_inline)) {
    const uint32_t *sc = ssc[g & 1];
#pragma unroll
    for (int i = 0; i < TMW; ++i) scA[i] = sc[(wm * TMW + i) * 64 + lane];
#pragma unroll
    for (int j = 0; j < TNW; ++j) scB[j] = sc[(AT + wn * TNW + j) * 64 + lane];
    if (g + 1 < KS4) issue_scales(g + 1);
  };
  const int G = KS / 4;                                  // whole groups of four k-steps
  for (int g = 0; g < G; ++g) {
    uint32_t scA[TMW], scB[TNW];
    group_scales(g, scA, scB);
    step(std::integral_constant<int, 0>{}, 4 * g, scA, scB);
    step(std::integral_constant<int, 1>{}, 4 * g + 1, scA, scB);
    step(std::integral_constant<int, 2>{}, 4 * g + 2, scA, scB);
    step(std::integral_constant<int, 3>{}, 4 * g + 3, scA, scB);
  }
  if (const int rem = KS - 4 * G; rem > 0) {             // the last group's 1 .. 3 k-steps
    uint32_t scA[TMW], scB[TNW];
    group_scales(G, scA, scB);
    step(std::integral_constant<int, 0>{}, 4 * G, scA, scB);
    if (rem > 1) step(std::integral_constant<int, 1>{}, 4 * G + 1, scA, scB);
    if (rem > 2) step(std::integral_constant<int, 2>{}, 4 * G + 2, scA, scB);
  }

  // epilogue: Y = acc + U L2 + bias; per row tile the wave's 16 x WCOL
  // values go through a wave-private LDS region of the stage buffers and
  // leave as 16-byte row-contiguous stores
  constexpr int WCOL = TNW * 16;
  static_assert(WGM * WGN * 16 * WCOL * 4 <= (int)sizeof(ops), "transpose region");
  char *tbuf = reinterpret_cast<char *>(&ops[0]) + wave * (16 * WCOL * 4);
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
        for (int c = 0; c < RPT; ++c) y = __builtin_fmaf(eu[c * BMR + rr], el2[c * BNC + cc], y);
        y += eb[cc];
        const int off = (rowq + qq) * WCOL + j * 16 + colq;
        if (a.y_bf16)
          reinterpret_cast<uint16_t *>(tbuf)[off] = f32_to_bf16(y);
        else
          reinterpret_cast<float *>(tbuf)[off] = y;
      }
    }
    const int mrow0 = (mt0 + wm * TMW + i) * 16;
    for (int k = lane; k < 16 * cpr; k += 64) {
      const int row = k / cpr, ch = k % cpr;
      const int m = mrow0 + row, n = ncol0 + ch * per16;
      if (m >= a.M || n >= a.N) continue;
      const v4u v = *reinterpret_cast<const v4u *>(tbuf + (row * WCOL + ch * per16) * yb);
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

// Workgroup shape.  128 x 128 (2 x 4 waves of 64 x 32) and, for rank up
// to 4, 128 x 256 (2 x 4 waves of 64 x 64); two workgroups per CU either
// way.  Measured with the register-staged loads of an earlier version
// against 2 x 2 waves of 64 x 64 (248 VGPRs, two waves per SIMD): 13 %
// faster at pixart size, 8 % on the FLUX and Qwen3 up layers; a 256 x 128
// workgroup ran at one wave per SIMD and was slower.  The wide tile does a
// k-step's MFMAs with a third fewer LDS operand reads, but has half as many
// workgroups to spread over the CUs.  Model, in the time a CU running two
// 128 x 128 workgroups takes per k-step: 2.0 per 128 x 128 tile pair-wise,
// 1.4 for one alone on its CU, and 1.25 times faster per output for the wide
// tile (3.2 and 2.24 per wide tile); workgroups fill the CUs in rounds of
// two per CU, a last round of at most one per CU runs at the lone rate.
// Fitted to FLUX.1 up and down, Qwen3 up and down at 256 and 2048 tokens,
// SANA QKV and pixart, where it picks the faster shape on each; the wide
// shape must win by 2 %.
double mx_rounds_time(long long tiles, double pair, double alone) {
  const long long slots = 2LL * kMxCUs, full = tiles / slots, rest = tiles % slots;
  return (double)full * pair + (rest == 0 ? 0.0 : rest <= kMxCUs ? alone : pair);
}

bool mx_wide(int M, int N, int r) {
  if (r > 4) return false;    // the wide kernel keeps its epilogue operands for rank <= 4 only
  const long long mblk = ceil_div(M, 128);
  const double narrow = mx_rounds_time(ceil_div(N, 128) * mblk, 2.0, 1.4);
  const double wide = mx_rounds_time(ceil_div(N, 256) * mblk, 3.2, 2.24);
  return wide < 0.98 * narrow;
}

template <int RP>
hipError_t launch_mx_gemm(const MxArgs &a, hipStream_t s) {
  if constexpr (RP <= 4) {
    if (mx_wide(a.M, a.N, a.r)) {
      const int tiles = ceil_div(a.N, 256) * ceil_div(a.M, 128);
      hipLaunchKernelGGL((k_mx_gemm_w<RP>), dim3((unsigned)tiles), dim3(512), 0, s, a);
      return hipGetLastError();
    }
  }
  const int tiles = ceil_div(a.N, 128) * ceil_div(a.M, 128);
  hipLaunchKernelGGL((k_mx_gemm<RP>), dim3((unsigned)tiles), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int RP>
hipError_t launch_mx_rp(const MxArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_mx_quant<RP>, dim3((unsigned)(a.Mpad / 16), (unsigned)a.u_slices), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_mx_gemm<RP>(a, s);
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

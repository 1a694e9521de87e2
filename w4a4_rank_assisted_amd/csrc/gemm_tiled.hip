// gemm_tiled.hip -- K2 (TILED): the int4 x int4 residual contraction with an
// int32 partial sum per 64-wide group, rescaled by sx * sw in fp32, plus the
// rank-r epilogue U * L2 + bias.
//
// Operation (hsq.h formula block; W ~ L1*L2 + Q(R), Deflating the Hessian,
// abstract; group-64, Table 1 caption).
//
// One 16x16x64 int8 MFMA covers exactly one group of one 16x16 output tile.
// Operands: A = activation codes (int8, written by K1 in MFMA lane order),
// B = residual codes unpacked from nibbles to 16*code while staging to LDS,
// so the MFMA yields 16*P.  The MFMA accumulator input is the bit pattern of
// 1.5*2^23; the result bits then read as the float 1.5*2^23 + 16P exactly,
// and two FMAs per element finish the group:
//   u   = fma(D, sw, -1.5*2^23*sw)   (= 16P*sw rounded once; the constant
//                                      product is exact: 3*2^22 * fp16)
//   acc = fma(u, sx/16, acc)
//
// Workgroup: 256 threads = 4 waves in 2x2, tile BM x BN; each wave owns
// (BM/2) x (BN/2) = TM x TN MFMA tiles.  K advances two groups per stage;
// stages are double-buffered in LDS with register prefetch, one barrier per
// stage.
#include "hsq_internal.h"

namespace hsq {

namespace {

constexpr uint32_t kNibMask = 0xF0F0F0F0u;

template <int BM, int BN>
struct Smem {
  static constexpr int TMB = BM / 16, TNB = BN / 16;
  int8_t a[2][TMB][2][64][16];      // [buf][m-tile][group][lane][bytes]
  int8_t b[2][2][TNB][64][16];      // [buf][group][n-tile][lane][bytes]
  float2 sw[2][2][BN];              // [buf][group][col] = (sw, -magic*sw)
  float sx[2][TMB][2][16];          // [buf][m-tile][group][row]
};

template <int BM, int BN, bool DUMP>
__global__ __launch_bounds__(256, 2) void k_gemm_tiled(GemmArgs a) {
  constexpr int TMB = BM / 16, TNB = BN / 16;
  constexpr int TM = TMB / 2, TN = TNB / 2;        // per wave
  constexpr int A_ITERS = TMB * 2 * 64 / 256;      // 16-byte chunks per thread
  constexpr int B_ITERS = TNB * 64 / 256;
  static_assert(A_ITERS >= 1 && B_ITERS >= 1, "tile too small");
  static_assert(2 * BN == 256 && TMB * 32 == 256, "scale staging assumes BM = BN = 128");
  __shared__ Smem<BM, BN> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int proj = blockIdx.z;
  const int mt0 = blockIdx.y * TMB;                 // first m-tile of this block
  const int nt0 = blockIdx.x * TNB;
  const int MT = a.Mpad / 16, NT = (a.N + 15) / 16;
  const int GP = a.Gp / 2;
  const uint8_t *w = a.w + (size_t)proj * a.w_stride;
  const uint16_t *sw = a.sw + (size_t)proj * a.G * a.N;
  if (DUMP && ((mt0 + TMB) * 16 <= a.m0 || mt0 * 16 >= a.m0 + a.mc ||
               (nt0 + TNB) * 16 <= a.n0 || nt0 * 16 >= a.n0 + a.nc))
    return;  // whole block outside the window (uniform: before any barrier)

  uint4 ra[A_ITERS], rb[B_ITERS];
  float rsw, rsx;

  auto load_stage = [&](int gp) {
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      int c = i * 256 + tid;
      int mi = c >> 7, rem = c & 127;
      ra[i] = (mt0 + mi < MT)
                  ? *reinterpret_cast<const uint4 *>(
                        a.qa + ((size_t)(mt0 + mi) * a.Gp + 2 * gp) * 1024 + (size_t)rem * 16)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      int c = i * 256 + tid;
      int ni = c >> 6, l = c & 63;
      rb[i] = (nt0 + ni < NT)
                  ? *reinterpret_cast<const uint4 *>(
                        w + ((size_t)(nt0 + ni) * GP + gp) * 1024 + (size_t)l * 16)
                  : make_uint4(0, 0, 0, 0);
    }
    {
      int gg = tid / BN, col = tid % BN;
      int g = 2 * gp + gg, n = nt0 * 16 + col;
      rsw = (g < a.G && n < a.N) ? f16_to_f32(sw[(size_t)g * a.N + n]) : 0.0f;
    }
    {
      int mi = tid >> 5, rem = tid & 31;
      rsx = (mt0 + mi < MT) ? a.sxs[((size_t)(mt0 + mi) * a.Gp + 2 * gp) * 16 + rem] : 0.0f;
    }
  };

  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      int c = i * 256 + tid;
      int mi = c >> 7, rem = c & 127;
      *reinterpret_cast<uint4 *>(&sm.a[buf][mi][rem >> 6][rem & 63][0]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      int c = i * 256 + tid;
      int ni = c >> 6, l = c & 63;
      uint4 v = rb[i];
      uint4 g0 = make_uint4(v.x & kNibMask, (v.x << 4) & kNibMask, v.y & kNibMask,
                            (v.y << 4) & kNibMask);
      uint4 g1 = make_uint4(v.z & kNibMask, (v.z << 4) & kNibMask, v.w & kNibMask,
                            (v.w << 4) & kNibMask);
      *reinterpret_cast<uint4 *>(&sm.b[buf][0][ni][l][0]) = g0;
      *reinterpret_cast<uint4 *>(&sm.b[buf][1][ni][l][0]) = g1;
    }
    {
      int gg = tid / BN, col = tid % BN;
      sm.sw[buf][gg][col] = make_float2(rsw, -kMagic * rsw);
    }
    {
      int mi = tid >> 5, rem = tid & 31;
      sm.sx[buf][mi][rem >> 4][rem & 15] = rsx;
    }
  };

  float acc[TM][TN][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][j][q] = 0.0f;

  const v4i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
  const int rowq = 4 * (lane >> 4);   // first of the 4 rows this lane holds
  const int colq = lane & 15;

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int gp = 0; gp < GP; ++gp) {
    const int buf = gp & 1;
    if (gp + 1 < GP) load_stage(gp + 1);

#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      v4i av[TM], bv[TN];
      float4 sxv[TM];
      float2 swv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        av[i] = *reinterpret_cast<const v4i *>(&sm.a[buf][wm * TM + i][gg][lane][0]);
        sxv[i] = *reinterpret_cast<const float4 *>(&sm.sx[buf][wm * TM + i][gg][rowq]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        bv[j] = *reinterpret_cast<const v4i *>(&sm.b[buf][gg][wn * TN + j][lane][0]);
        swv[j] = sm.sw[buf][gg][(wn * TN + j) * 16 + colq];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], bv[j], magic, 0, 0, 0);
          if (DUMP) {
            const int g = 2 * gp + gg;
            const int n = (nt0 + wn * TN + j) * 16 + colq;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int m = (mt0 + wm * TM + i) * 16 + rowq + q;
              if (g < a.G && m >= a.m0 && m < a.m0 + a.mc && n >= a.n0 && n < a.n0 + a.nc)
                a.P[((size_t)(m - a.m0) * a.nc + (n - a.n0)) * a.G + g] = (d[q] - kMagicBits) >> 4;
            }
          } else {
            const float s0 = sxv[i].x, s1 = sxv[i].y, s2 = sxv[i].z, s3 = sxv[i].w;
            float u;
            u = __builtin_fmaf(__int_as_float(d[0]), swv[j].x, swv[j].y);
            acc[i][j][0] = __builtin_fmaf(u, s0, acc[i][j][0]);
            u = __builtin_fmaf(__int_as_float(d[1]), swv[j].x, swv[j].y);
            acc[i][j][1] = __builtin_fmaf(u, s1, acc[i][j][1]);
            u = __builtin_fmaf(__int_as_float(d[2]), swv[j].x, swv[j].y);
            acc[i][j][2] = __builtin_fmaf(u, s2, acc[i][j][2]);
            u = __builtin_fmaf(__int_as_float(d[3]), swv[j].x, swv[j].y);
            acc[i][j][3] = __builtin_fmaf(u, s3, acc[i][j][3]);
          }
        }
    }

    if (gp + 1 < GP) store_stage(buf ^ 1);
    __syncthreads();
  }

  if (DUMP) return;

  // ---- epilogue: Y = acc + U * L2 + bias ----
  const uint16_t *L2 = a.L2 ? a.L2 + (size_t)proj * a.r * a.N : nullptr;
  const uint16_t *bias = a.bias ? a.bias + (size_t)proj * a.N : nullptr;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int mrow = (mt0 + wm * TM + i) * 16 + rowq;  // rows mrow .. mrow+3
    if (mrow >= a.M) continue;
    float add[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) add[j][q] = 0.0f;
    for (int c = 0; c < a.r; ++c) {
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int sl = 0; sl < a.u_slices; ++sl) {
        const float4 v = *reinterpret_cast<const float4 *>(
            a.uw + ((size_t)sl * a.ucols + (size_t)proj * a.r + c) * a.Mpad + mrow);
        u.x += v.x; u.y += v.y; u.z += v.z; u.w += v.w;
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = (nt0 + wn * TN + j) * 16 + colq;
        const float l2 = n < a.N ? bf16_to_f32(L2[(size_t)c * a.N + n]) : 0.0f;
        add[j][0] = __builtin_fmaf(u.x, l2, add[j][0]);
        add[j][1] = __builtin_fmaf(u.y, l2, add[j][1]);
        add[j][2] = __builtin_fmaf(u.z, l2, add[j][2]);
        add[j][3] = __builtin_fmaf(u.w, l2, add[j][3]);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = (nt0 + wn * TN + j) * 16 + colq;
      if (n >= a.N) continue;
      const float bb = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = mrow + q;
        if (m >= a.M) break;
        const float y = acc[i][j][q] + add[j][q] + bb;
        const size_t off = ((size_t)proj * a.M + m) * a.N + n;
        if (a.y_bf16)
          reinterpret_cast<uint16_t *>(a.Y)[off] = f32_to_bf16(y);
        else
          reinterpret_cast<float *>(a.Y)[off] = y;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  if (dump) {
    // blocks up to the last one touching the window; the others exit at once
    dim3 grid((unsigned)((a.n0 + a.nc - 1) / BN + 1), (unsigned)((a.m0 + a.mc - 1) / BM + 1), 1u);
    hipLaunchKernelGGL((k_gemm_tiled<BM, BN, true>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid((unsigned)ceil_div(a.N, BN), (unsigned)ceil_div(a.M, BM), (unsigned)batch);
  hipLaunchKernelGGL((k_gemm_tiled<BM, BN, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hsq

// gemm_skinny.hip -- K2 (SKINNY): the residual contraction for small token
// counts (M <= 64), where the layer is bound by streaming the packed weights
// from HBM (K*N/2 bytes for 2*M*N*K operations).
//
// Same arithmetic as the tiled kernel (hsq.h formula block; one 16x16x64
// int8 MFMA per group and output tile, magic-constant accumulator, two FMAs
// per element and group).  Mapping: a workgroup owns one 16-column tile of
// one projection; its W waves split the K groups into contiguous ranges, so
// every weight byte is loaded by exactly one lane, straight from HBM into
// registers with 16-byte loads, several group pairs in flight per lane.
// The activation codes (M*K bytes) are small and served from L2.  The W
// partial tiles are summed through LDS in wave order (deterministic), and
// the epilogue adds U * L2 and the bias -- no split-K buffer, one launch.
#include "hsq_internal.h"

namespace hsq {

namespace {

constexpr uint32_t kNibMask = 0xF0F0F0F0u;

template <int MT, bool DUMP>
__global__ __launch_bounds__(512) void k_gemm_skinny(GemmArgs a, int W) {
  // dynamic LDS: partial tiles [W][MT][4][64], then U [r][16*MT] (slices
  // summed), L2 [r][16], bias [16]
  extern __shared__ float red[];
  float *eu = red + W * MT * 4 * 64;
  float *el2 = eu + a.r * MT * 16;
  float *eb = el2 + a.r * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nt = blockIdx.x + (DUMP ? a.n0 / 16 : 0);
  const int proj = blockIdx.y;
  const int GP = a.Gp / 2;
  const int per = (GP + W - 1) / W;
  const int gp0 = wave * per;
  const int gp1 = min(GP, gp0 + per);
  const int colq = lane & 15, rowq = 4 * (lane >> 4);
  const int n = nt * 16 + colq;
  const bool ncol = n < a.N;
  const uint8_t *wp = a.w + (size_t)proj * a.w_stride + (size_t)nt * GP * 1024 + (size_t)lane * 16;
  const uint16_t *swp = a.sw ? a.sw + (size_t)proj * a.G * a.N + (ncol ? n : 0) : nullptr;
  const v4i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};

  // epilogue operands into LDS first (their loads overlap the weight stream;
  // the barrier before the epilogue orders them)
  if (!DUMP) {
    const int nthr = W * 64;
    for (int p = tid; p < a.r * MT * 16; p += nthr) {
      const int c = p / (MT * 16), row = p % (MT * 16);
      float u = 0.0f;
#pragma unroll
      for (int sl = 0; sl < kMaxUSlices; ++sl) {
        const float v = a.uw[((size_t)min(sl, a.u_slices - 1) * a.ucols + (size_t)proj * a.r + c) * a.Mpad + row];
        u += sl < a.u_slices ? v : 0.0f;
      }
      for (int sl = kMaxUSlices; sl < a.u_slices; ++sl)
        u += a.uw[((size_t)sl * a.ucols + (size_t)proj * a.r + c) * a.Mpad + row];
      eu[c * MT * 16 + row] = u;
    }
    for (int p = tid; p < a.r * 16; p += nthr) {
      const int c = p / 16, col = p % 16;
      el2[p] = bf16_to_f32(a.L2[((size_t)proj * a.r + c) * a.N + min(nt * 16 + col, a.N - 1)]);
    }
    if (tid < 16)
      eb[tid] = a.bias ? bf16_to_f32(a.bias[(size_t)proj * a.N + min(nt * 16 + tid, a.N - 1)]) : 0.0f;
  }

  float acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;

  // prefetch ring: D group pairs of weights, weight scales, activation
  // codes and activation scales in flight per lane (D = 4 / MT registers
  // budget); every operand of a group pair is loaded D pairs ahead
  constexpr int D = MT == 1 ? 4 : (MT == 2 ? 2 : 1);
  v4u wbuf[D];
  uint32_t sbuf[D];
  v4i abuf[D][MT][2];
  v4f xbuf[D][MT][2];
  auto fetch = [&](int gp, int u) __attribute__((always_inline)) {
    wbuf[u] = *reinterpret_cast<const v4u *>(wp + (size_t)gp * 1024);
    sbuf[u] = 0;
    if (!DUMP && ncol) {
      const int g = 2 * gp;
      const uint32_t lo = swp[(size_t)g * a.N];
      const uint32_t hi = (g + 1 < a.G) ? swp[(size_t)(g + 1) * a.N] : 0u;
      sbuf[u] = lo | (hi << 16);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * gp + h;
        abuf[u][i][h] = *reinterpret_cast<const v4i *>(a.qa + (((size_t)i * a.Gp + g) * 64 + lane) * 16);
        if (!DUMP)
          xbuf[u][i][h] = *reinterpret_cast<const v4f *>(a.sxs + ((size_t)i * a.Gp + g) * 16 + rowq);
      }
  };
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (gp0 + u < gp1) fetch(gp0 + u, u);

  for (int base = gp0; base < gp1; base += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int gp = base + u;
      if (gp >= gp1) break;
      const v4u wv = wbuf[u];
      const uint32_t sv = sbuf[u];
      v4i av[MT][2];
      v4f sx[MT][2];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          av[i][h] = abuf[u][i][h];
          sx[i][h] = xbuf[u][i][h];
        }
      if (gp + D < gp1) fetch(gp + D, u);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * gp + h;
        const uint32_t w0 = h ? wv.z : wv.x, w1 = h ? wv.w : wv.y;
        const v4i b = {(int)(w0 & kNibMask), (int)((w0 << 4) & kNibMask), (int)(w1 & kNibMask),
                       (int)((w1 << 4) & kNibMask)};
        const float swf = f16_to_f32((uint16_t)(h ? sv >> 16 : sv & 0xFFFFu));
        const float nsw = -kMagic * swf;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i][h], b, magic, 0, 0, 0);
          if (DUMP) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int m = i * 16 + rowq + q;
              if (g < a.G && m >= a.m0 && m < a.m0 + a.mc && n >= a.n0 && n < a.n0 + a.nc)
                a.P[((size_t)(m - a.m0) * a.nc + (n - a.n0)) * a.G + g] = (d[q] - kMagicBits) >> 4;
            }
          } else {
            float t;
            t = __builtin_fmaf(__int_as_float(d[0]), swf, nsw);
            acc[i][0] = __builtin_fmaf(t, sx[i][h][0], acc[i][0]);
            t = __builtin_fmaf(__int_as_float(d[1]), swf, nsw);
            acc[i][1] = __builtin_fmaf(t, sx[i][h][1], acc[i][1]);
            t = __builtin_fmaf(__int_as_float(d[2]), swf, nsw);
            acc[i][2] = __builtin_fmaf(t, sx[i][h][2], acc[i][2]);
            t = __builtin_fmaf(__int_as_float(d[3]), swf, nsw);
            acc[i][3] = __builtin_fmaf(t, sx[i][h][3], acc[i][3]);
          }
        }
      }
    }
  }
  if (DUMP) return;

  // ---- ordered reduction of the W partial tiles, then the epilogue ----
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[((wave * MT + i) * 4 + q) * 64 + lane] = acc[i][q];
  __syncthreads();

  for (int i = wave; i < MT; i += W) {
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    for (int v = 0; v < W; ++v)
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] += red[((v * MT + i) * 4 + q) * 64 + lane];
    const int mrow = i * 16 + rowq;
    if (!ncol || mrow >= a.M) continue;
    for (int c = 0; c < a.r; ++c) {
      const float l2 = el2[c * 16 + colq];
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = __builtin_fmaf(eu[c * MT * 16 + mrow + q], l2, y[q]);
    }
    const float bb = eb[colq];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = mrow + q;
      if (m >= a.M) break;
      const size_t off = ((size_t)proj * a.M + m) * a.N + n;
      if (a.y_bf16)
        reinterpret_cast<uint16_t *>(a.Y)[off] = f32_to_bf16(y[q] + bb);
      else
        reinterpret_cast<float *>(a.Y)[off] = y[q] + bb;
    }
  }
}

template <int MT>
hipError_t launch_mt(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  const int NT = ceil_div(a.N, kTile), GP = a.Gp / 2;
  // waves per workgroup: enough to put ~4 waves on every SIMD of the chip
  int W = ceil_div(4096, NT * batch);
  if (W > 8) W = 8;
  if (W > GP) W = GP;
  if (W < 1) W = 1;
  const size_t lds = ((size_t)W * MT * 4 * 64 + (size_t)a.r * MT * 16 + (size_t)a.r * 16 + 16) * sizeof(float);
  if (dump) {
    const int nt0 = a.n0 / 16, nt1 = (a.n0 + a.nc - 1) / 16;
    hipLaunchKernelGGL((k_gemm_skinny<MT, true>), dim3((unsigned)(nt1 - nt0 + 1), 1u),
                       dim3((unsigned)(64 * W)), 0, s, a, W);
  } else {
    hipLaunchKernelGGL((k_gemm_skinny<MT, false>), dim3((unsigned)NT, (unsigned)batch),
                       dim3((unsigned)(64 * W)), lds, s, a, W);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  switch (ceil_div(a.M, kTile)) {
    case 1: return launch_mt<1>(a, batch, dump, s);
    case 2: return launch_mt<2>(a, batch, dump, s);
    case 3: return launch_mt<3>(a, batch, dump, s);
    case 4: return launch_mt<4>(a, batch, dump, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hsq

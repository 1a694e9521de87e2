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
constexpr int kDepth = 4;  // group pairs of weights in flight per lane

template <int MT, bool DUMP>
__global__ __launch_bounds__(1024) void k_gemm_skinny(GemmArgs a, int W) {
  extern __shared__ float red[];  // [W][MT][4][64]
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

  float acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;

  uint4 wbuf[kDepth];
  uint32_t sbuf[kDepth];
  auto fetch = [&](int gp, uint4 &wv, uint32_t &sv) {
    wv = *reinterpret_cast<const uint4 *>(wp + (size_t)gp * 1024);
    sv = 0;
    if (!DUMP && ncol) {
      const int g = 2 * gp;
      uint32_t lo = swp[(size_t)g * a.N];
      uint32_t hi = (g + 1 < a.G) ? swp[(size_t)(g + 1) * a.N] : 0u;
      sv = lo | (hi << 16);
    }
  };
#pragma unroll
  for (int u = 0; u < kDepth; ++u)
    if (gp0 + u < gp1) fetch(gp0 + u, wbuf[u], sbuf[u]);

  for (int base = gp0; base < gp1; base += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int gp = base + u;
      if (gp >= gp1) break;
      const uint4 wv = wbuf[u];
      const uint32_t sv = sbuf[u];
      if (gp + kDepth < gp1) fetch(gp + kDepth, wbuf[u], sbuf[u]);
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
          const v4i av = *reinterpret_cast<const v4i *>(
              a.qa + (((size_t)i * a.Gp + g) * 64 + lane) * 16);
          const v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, b, magic, 0, 0, 0);
          if (DUMP) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int m = i * 16 + rowq + q;
              if (g < a.G && m >= a.m0 && m < a.m0 + a.mc && n >= a.n0 && n < a.n0 + a.nc)
                a.P[((size_t)(m - a.m0) * a.nc + (n - a.n0)) * a.G + g] = (d[q] - kMagicBits) >> 4;
            }
          } else {
            const float4 sx = *reinterpret_cast<const float4 *>(
                a.sxs + ((size_t)i * a.Gp + g) * 16 + rowq);
            float t;
            t = __builtin_fmaf(__int_as_float(d[0]), swf, nsw);
            acc[i][0] = __builtin_fmaf(t, sx.x, acc[i][0]);
            t = __builtin_fmaf(__int_as_float(d[1]), swf, nsw);
            acc[i][1] = __builtin_fmaf(t, sx.y, acc[i][1]);
            t = __builtin_fmaf(__int_as_float(d[2]), swf, nsw);
            acc[i][2] = __builtin_fmaf(t, sx.z, acc[i][2]);
            t = __builtin_fmaf(__int_as_float(d[3]), swf, nsw);
            acc[i][3] = __builtin_fmaf(t, sx.w, acc[i][3]);
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

  const uint16_t *L2 = a.L2 ? a.L2 + (size_t)proj * a.r * a.N : nullptr;
  const uint16_t *bias = a.bias ? a.bias + (size_t)proj * a.N : nullptr;
  for (int i = wave; i < MT; i += W) {
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    for (int v = 0; v < W; ++v)
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] += red[((v * MT + i) * 4 + q) * 64 + lane];
    const int mrow = i * 16 + rowq;
    if (!ncol || mrow >= a.M) continue;
    for (int c = 0; c < a.r; ++c) {
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int sl = 0; sl < a.u_slices; ++sl) {
        const float4 v = *reinterpret_cast<const float4 *>(
            a.uw + ((size_t)sl * a.ucols + (size_t)proj * a.r + c) * a.Mpad + mrow);
        u.x += v.x; u.y += v.y; u.z += v.z; u.w += v.w;
      }
      const float l2 = bf16_to_f32(L2[(size_t)c * a.N + n]);
      y[0] = __builtin_fmaf(u.x, l2, y[0]);
      y[1] = __builtin_fmaf(u.y, l2, y[1]);
      y[2] = __builtin_fmaf(u.z, l2, y[2]);
      y[3] = __builtin_fmaf(u.w, l2, y[3]);
    }
    const float bb = bias ? bf16_to_f32(bias[n]) : 0.0f;
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
  if (W > 16) W = 16;
  if (W > GP) W = GP;
  if (W < 1) W = 1;
  const size_t lds = (size_t)W * MT * 4 * 64 * sizeof(float);
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

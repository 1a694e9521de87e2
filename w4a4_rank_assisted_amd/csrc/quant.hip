// quant.hip -- K1: one pass over X that smooths it, quantizes it per token in
// 64-wide groups to symmetric int4, and accumulates the rank-r down
// projection U = xh * L1 of the smoothed, unquantized activations.
//
// Operation (hsq.h formula block): smoothing by a diagonal scale (H-SVDQuant
// explainer, rit.work, section on Hessian deflation), group-64 4-bit
// activations (Deflating the Hessian, Table 1 caption), high-precision
// branch on unquantized inputs (DiRotQ notes, key design 2).
//
// Mapping: one lane per (token, 64-channel group).  A lane loads its group
// with eight 16-byte loads, finds the absmax in registers, computes the fp16
// scale and its reciprocal once, writes the codes, and forms its group's
// share of U.  A wave holds 16 tokens x 4 groups, so lanes that share a group
// read the same 1/lambda (LDS) and L1 (cache) addresses; a workgroup of 256
// lanes owns R tokens x (256/R) group slots and loops its lanes over the
// K-slice's groups.  It computes 1/lambda for the slice's channels into LDS
// (exact IEEE division) and sums the U shares of each token through LDS in a
// fixed order.  Large K is split into at most four K-slices, whose U
// partials the consumer sums.  The pass is HBM-bound: X is read once, codes
// and scales are written once.
#include "hsq_internal.h"

namespace hsq {

namespace {

constexpr int kSliceGroups = 64;      // groups per K-slice of the internal pass

template <int NR, bool PUB>
__global__ __launch_bounds__(256) void k_quant(QuantArgs a, int ng, int R) {
  // dynamic LDS: 1/lambda of the slice's channels, then the U shares
  extern __shared__ float lds[];
  float *inv_lam = lds;                           // ng * 64
  float *upart = lds + ng * kGroup;               // NR * 256

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int WR = R / 16;                          // waves along the token axis
  const int GW = 256 / R;                         // group slots of the workgroup
  const int rl = (lane & 15) + 16 * (wave % WR);  // token of this lane
  const int gs = (lane >> 4) + 4 * (wave / WR);   // group slot of this lane
  const int gend = a.kend / kGroup;               // groups to write (G or Gp)
  const int gb = blockIdx.y * ng;                 // first group of the slice
  const int gn = min(ng, gend - gb);              // groups in this slice
  const int m = blockIdx.x * R + rl;
  const int mrows = PUB ? a.M : a.Mpad;           // rows this pass writes

  for (int i = tid; i < gn * kGroup; i += 256) {
    const int k = gb * kGroup + i;
    inv_lam[i] = (k < a.K) ? 1.0f / f16_to_f32(a.lam[k]) : 0.0f;
  }
  __syncthreads();

  float acc[NR > 0 ? NR : 1];
#pragma unroll
  for (int c = 0; c < (NR > 0 ? NR : 1); ++c) acc[c] = 0.0f;

  if (m < mrows) {
    for (int gi = gs; gi < gn; gi += GW) {
      const int g = gb + gi;
      const bool in = m < a.M && g < a.G;         // outside: pad row / group, zeros
      float xh[kGroup];
      {
        v4u raw[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          raw[t] = in ? *reinterpret_cast<const v4u *>(a.X + (size_t)m * a.K + (size_t)g * kGroup + 8 * t)
                      : (v4u){0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const int i = 8 * t + 2 * h;
            xh[i] = bf16_to_f32(raw[t][h] & 0xFFFFu) * inv_lam[gi * kGroup + i];
            xh[i + 1] = bf16_to_f32(raw[t][h] >> 16) * inv_lam[gi * kGroup + i + 1];
          }
      }

      if (a.write_codes) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) amax = fmaxf(amax, fabsf(xh[i]));
        uint16_t s16 = 0;
        if (amax != 0.0f) {
          s16 = f32_to_f16(amax / 7.0f);
          if (s16 == 0x7C00u) s16 = 0x7BFFu;      // saturate at 65504
        }
        const float s = f16_to_f32(s16);
        const float inv_s = (s16 != 0) ? 1.0f / s : 0.0f;
        uint32_t w[16];                           // 64 codes: int8 (internal) / nibbles (public)
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = 0;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
          const float t = __builtin_rintf(xh[i] * inv_s);  // ties to even
          const int q = (int)fminf(fmaxf(t, -8.0f), 7.0f);
          if (PUB)
            w[i >> 3] |= (uint32_t)(q & 0xF) << (4 * (i & 7));
          else
            w[i >> 2] |= (uint32_t)(q & 0xFF) << (8 * (i & 3));
        }
        if (PUB) {
          if (in) {
            v4u *dst = reinterpret_cast<v4u *>(a.qx + (size_t)m * (a.K / 2) + (size_t)g * 32);
            dst[0] = (v4u){w[0], w[1], w[2], w[3]};
            dst[1] = (v4u){w[4], w[5], w[6], w[7]};
            a.sx[(size_t)m * a.G + g] = s16;
          }
        } else {
          // MFMA A-operand order: lane slot (m % 16) + 16 * kq holds
          // channels 64g + 16kq .. +15 of row m
          const int mt = m >> 4;
          int8_t *base = a.qa + ((size_t)mt * a.Gp + g) * 1024 + (size_t)(m & 15) * 16;
#pragma unroll
          for (int kq = 0; kq < 4; ++kq)
            *reinterpret_cast<v4u *>(base + kq * 256) =
                (v4u){w[4 * kq], w[4 * kq + 1], w[4 * kq + 2], w[4 * kq + 3]};
          a.sxs[((size_t)mt * a.Gp + g) * 16 + (m & 15)] = s * 0.0625f;
        }
      }

      if (NR > 0 && in) {
        // this group's share of U for rank columns c0 .. c0+cb-1
        if ((a.r & 3) == 0) {
          // four columns of one projection per 8-byte L1 row chunk
#pragma unroll
          for (int c = 0; c < NR; c += 4) {
            if (c >= a.cb) break;
            const int cc = a.c0 + c, b = cc / a.r, j = cc % a.r;
            const uint16_t *l1 = a.L1 + ((size_t)b * a.K + (size_t)g * kGroup) * a.r + j;
            float s0 = acc[c], s1 = acc[c + 1], s2 = acc[c + 2], s3 = acc[c + 3];
#pragma unroll
            for (int i0 = 0; i0 < kGroup; i0 += 16) {
#pragma unroll
              for (int i = i0; i < i0 + 16; ++i) {
                const v2u v = *reinterpret_cast<const v2u *>(l1 + (size_t)i * a.r);
                s0 = __builtin_fmaf(xh[i], bf16_to_f32(v.x & 0xFFFFu), s0);
                s1 = __builtin_fmaf(xh[i], bf16_to_f32(v.x >> 16), s1);
                s2 = __builtin_fmaf(xh[i], bf16_to_f32(v.y & 0xFFFFu), s2);
                s3 = __builtin_fmaf(xh[i], bf16_to_f32(v.y >> 16), s3);
              }
              // at most 16 L1 loads in flight: no load moves across this
              asm volatile("" : "+v"(s0), "+v"(s1), "+v"(s2), "+v"(s3) : : "memory");
            }
            acc[c] = s0; acc[c + 1] = s1; acc[c + 2] = s2; acc[c + 3] = s3;
          }
        } else {
#pragma unroll
          for (int c = 0; c < NR; ++c) {
            if (c >= a.cb) break;
            const int cc = a.c0 + c, b = cc / a.r, j = cc % a.r;
            const uint16_t *l1 = a.L1 + ((size_t)b * a.K + (size_t)g * kGroup) * a.r + j;
            float sacc = acc[c];
#pragma unroll
            for (int i0 = 0; i0 < kGroup; i0 += 16) {
#pragma unroll
              for (int i = i0; i < i0 + 16; ++i)
                sacc = __builtin_fmaf(xh[i], bf16_to_f32(l1[(size_t)i * a.r]), sacc);
              asm volatile("" : "+v"(sacc) : : "memory");
            }
            acc[c] = sacc;
          }
        }
      }
    }
  }

  if (NR > 0) {
    // sum the shares of each token over its group slots (fixed order)
#pragma unroll
    for (int c = 0; c < NR; ++c) upart[(c * GW + gs) * R + rl] = acc[c];
    __syncthreads();
    for (int p = tid; p < R * a.cb; p += 256) {
      const int r0 = p % R, c = p / R;
      const int mm = blockIdx.x * R + r0;
      if (mm >= mrows) continue;
      float s = 0.0f;
      for (int q = 0; q < GW; ++q) s += upart[(c * GW + q) * R + r0];
      if (PUB)
        a.u_pub[(size_t)mm * a.r + a.c0 + c] = s;
      else
        a.uw[((size_t)blockIdx.y * a.ucols + a.c0 + c) * a.Mpad + mm] = s;
    }
  }
}

template <bool PUB>
hipError_t launch_variant(const QuantArgs &a, dim3 grid, int ng, int R, hipStream_t s) {
  const int cb = a.cb;
  const int nr = cb == 0 ? 0 : cb <= 4 ? 4 : cb <= 8 ? 8 : cb <= 16 ? 16 : 32;
  const size_t lds = sizeof(float) * ((size_t)ng * kGroup + (size_t)256 * (nr ? nr : 1));
  switch (nr) {
    case 0: hipLaunchKernelGGL((k_quant<0, PUB>), grid, dim3(256), lds, s, a, ng, R); break;
    case 4: hipLaunchKernelGGL((k_quant<4, PUB>), grid, dim3(256), lds, s, a, ng, R); break;
    case 8: hipLaunchKernelGGL((k_quant<8, PUB>), grid, dim3(256), lds, s, a, ng, R); break;
    case 16: hipLaunchKernelGGL((k_quant<16, PUB>), grid, dim3(256), lds, s, a, ng, R); break;
    default: hipLaunchKernelGGL((k_quant<32, PUB>), grid, dim3(256), lds, s, a, ng, R); break;
  }
  return hipGetLastError();
}

}  // namespace

int quant_slices(int K) {
  const int s = ceil_div(padded_groups(K), kSliceGroups);
  return s < 1 ? 1 : (s > kMaxUSlices ? kMaxUSlices : s);
}

// One launch per block of up to 32 rank columns; codes and scales are
// written by the first.  `slices` K-slices (gridDim.y): 1 for the public
// pass, quant_slices(K) for the internal one.
hipError_t launch_quant(const QuantArgs &a0, int slices, hipStream_t s) {
  const bool pub = a0.qx != nullptr;
  const int gend = a0.kend / kGroup;
  const int ng = ceil_div(gend, slices);          // groups per slice
  if ((size_t)ng * kGroup * sizeof(float) > 96 * 1024) return hipErrorInvalidValue;
  // tokens per workgroup: 16 when the slice has many groups (16 group
  // slots), up to 64 for short slices (4 group slots)
  const int R = ng >= 12 ? 16 : (ng >= 6 ? 32 : 64);
  const int mrows = pub ? a0.M : a0.Mpad;
  dim3 grid((unsigned)ceil_div(mrows, R), (unsigned)slices);
  const int total = a0.r * a0.batch;
  int c0 = 0;
  do {
    QuantArgs a = a0;
    a.c0 = c0;
    a.cb = total - c0 < kRankBlock ? total - c0 : kRankBlock;
    a.write_codes = (c0 == 0);
    hipError_t e = pub ? launch_variant<true>(a, grid, ng, R, s)
                       : launch_variant<false>(a, grid, ng, R, s);
    if (e != hipSuccess) return e;
    c0 += kRankBlock;
  } while (c0 < total);
  return hipSuccess;
}

}  // namespace hsq

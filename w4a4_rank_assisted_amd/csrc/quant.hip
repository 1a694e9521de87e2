// quant.hip -- K1: one pass over X that smooths it, quantizes it per token in
// 64-wide groups to symmetric int4, and accumulates the rank-r down
// projection U = xh * L1 of the smoothed, unquantized activations.
//
// Operation (hsq.h formula block): smoothing by a diagonal scale (H-SVDQuant
// explainer, rit.work, section on Hessian deflation), group-64 4-bit
// activations (Deflating the Hessian, Table 1 caption), high-precision
// branch on unquantized inputs (DiRotQ notes, key design 2).
//
// Mapping: a workgroup of 4 waves owns 16 rows and one K-slice; wave w owns
// rows 16*bx + 4w .. +3.  In each 512-channel chunk lane l owns channels
// k = chunk + 8l .. +7 (one 128-bit load per row), so the 8 lanes 8i..8i+7
// hold one 64-wide group and reduce its absmax with three xor shuffles.
// 1/lambda is computed once per workgroup into LDS (exact IEEE division).
// The kernel is HBM-bound: X is read once, codes and scales written once.
#include "hsq_internal.h"

namespace hsq {

namespace {

constexpr int kLamTile = 4096;  // channels of 1/lambda kept in LDS at a time

__device__ __forceinline__ float group_absmax8(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  v = fmaxf(v, __shfl_xor(v, 2, 64));
  v = fmaxf(v, __shfl_xor(v, 4, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;  // identical on every lane: each step adds a commutative pair
}

// L1 values of channels k..k+7 for rank columns c..c+3 of the concatenated
// batch*r columns; zero beyond K or beyond the pass's columns.
__device__ __forceinline__ void load_l1_block(const QuantArgs &a, int k, int c, float (&l)[8][4]) {
  int cend = a.c0 + a.cb;
  if ((a.r & 3) == 0 && c + 3 < cend) {
    int b = c / a.r, j = c % a.r;  // four columns inside one projection
    const uint16_t *base = a.L1 + ((size_t)b * a.K + k) * a.r + j;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint2 v = *reinterpret_cast<const uint2 *>(base + (size_t)i * a.r);
      l[i][0] = bf16_to_f32(v.x & 0xFFFFu);
      l[i][1] = bf16_to_f32(v.x >> 16);
      l[i][2] = bf16_to_f32(v.y & 0xFFFFu);
      l[i][3] = bf16_to_f32(v.y >> 16);
    }
    return;
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    int cc = c + jj;
    bool ok = cc < cend;
    int b = ok ? cc / a.r : 0, j = ok ? cc % a.r : 0;
    const uint16_t *base = a.L1 + ((size_t)b * a.K + k) * a.r + j;
#pragma unroll
    for (int i = 0; i < 8; ++i) l[i][jj] = ok ? bf16_to_f32(base[(size_t)i * a.r]) : 0.0f;
  }
}

template <int NR, bool PUB>
__global__ __launch_bounds__(256) void k_quant(QuantArgs a) {
  __shared__ float inv_lam[kLamTile];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row0 = blockIdx.x * 16 + wave * 4;
  const int kbeg = blockIdx.y * a.kslice;
  const int kstop = min(kbeg + a.kslice, a.kend);

  float acc[4][NR > 0 ? NR : 1];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int c = 0; c < (NR > 0 ? NR : 1); ++c) acc[rr][c] = 0.0f;

  for (int sub = kbeg; sub < kstop; sub += kLamTile) {
    const int subend = min(sub + kLamTile, kstop);
    __syncthreads();  // previous tile fully consumed
    for (int i = tid; i < subend - sub; i += 256) {
      int k = sub + i;
      inv_lam[i] = (k < a.K) ? 1.0f / f16_to_f32(a.lam[k]) : 0.0f;
    }
    __syncthreads();

    for (int chunk = sub; chunk < subend; chunk += 512) {
      const int k = chunk + 8 * lane;
      if (k >= subend) continue;  // whole groups: subend is a multiple of 64
      const bool in_k = k < a.K;
      float inv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) inv[i] = inv_lam[k - sub + i];

      float xh[4][8];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int m = row0 + rr;
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (in_k && m < a.M) raw = *reinterpret_cast<const uint4 *>(a.X + (size_t)m * a.K + k);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xh[rr][2 * i] = bf16_to_f32(w[i] & 0xFFFFu) * inv[2 * i];
          xh[rr][2 * i + 1] = bf16_to_f32(w[i] >> 16) * inv[2 * i + 1];
        }
        if (!a.write_codes) continue;

        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(xh[rr][i]));
        amax = group_absmax8(amax);
        uint16_t s16 = 0;
        if (amax != 0.0f) {
          s16 = f32_to_f16(amax / 7.0f);
          if (s16 == 0x7C00u) s16 = 0x7BFFu;  // saturate at 65504
        }
        const float s = f16_to_f32(s16);
        const float inv_s = (s16 != 0) ? 1.0f / s : 0.0f;
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float t = __builtin_rintf(xh[rr][i] * inv_s);  // ties to even
          q[i] = (int)fminf(fmaxf(t, -8.0f), 7.0f);
        }
        const int g = k / kGroup;
        if (PUB) {
          if (in_k && m < a.M) {
            uint32_t packed = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
              packed |= (uint32_t)((q[2 * b] & 0xF) | ((q[2 * b + 1] & 0xF) << 4)) << (8 * b);
            *reinterpret_cast<uint32_t *>(a.qx + (size_t)m * (a.K / 2) + k / 2) = packed;
            if ((lane & 7) == 0) a.sx[(size_t)m * a.G + g] = s16;
          }
        } else {
          // m < Mpad always (grid covers the padded rows); k < 64*Gp
          const int mt = m >> 4;
          const int slot = (m & 15) + 16 * ((lane & 7) >> 1);
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            lo |= (uint32_t)(q[b] & 0xFF) << (8 * b);
            hi |= (uint32_t)(q[4 + b] & 0xFF) << (8 * b);
          }
          int8_t *dst = a.qa + (((size_t)mt * a.Gp + g) * 64 + slot) * 16 + 8 * (lane & 1);
          *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
          if ((lane & 7) == 0) a.sxs[((size_t)mt * a.Gp + g) * 16 + (m & 15)] = s * 0.0625f;
        }
      }

      if (NR > 0 && in_k) {
#pragma unroll
        for (int cb4 = 0; cb4 < NR / 4; ++cb4) {
          const int c = a.c0 + 4 * cb4;
          if (4 * cb4 >= a.cb) break;
          float l[8][4];
          load_l1_block(a, k, c, l);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              float s = acc[rr][4 * cb4 + jj];
#pragma unroll
              for (int i = 0; i < 8; ++i) s = __builtin_fmaf(xh[rr][i], l[i][jj], s);
              acc[rr][4 * cb4 + jj] = s;
            }
        }
      }
    }
  }

  if (NR > 0) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int m = row0 + rr;
#pragma unroll
      for (int c = 0; c < NR; ++c) {
        if (c >= a.cb) break;
        float v = wave_sum(acc[rr][c]);
        if (lane == (c & 63)) {
          if (PUB) {
            if (m < a.M) a.u_pub[(size_t)m * a.r + a.c0 + c] = v;
          } else {
            a.uw[((size_t)blockIdx.y * a.ucols + a.c0 + c) * a.Mpad + m] = v;
          }
        }
      }
    }
  }
}

template <bool PUB>
hipError_t launch_variant(const QuantArgs &a, dim3 grid, hipStream_t s) {
  int cb = a.cb;
  if (cb == 0)
    hipLaunchKernelGGL((k_quant<0, PUB>), grid, dim3(256), 0, s, a);
  else if (cb <= 4)
    hipLaunchKernelGGL((k_quant<4, PUB>), grid, dim3(256), 0, s, a);
  else if (cb <= 8)
    hipLaunchKernelGGL((k_quant<8, PUB>), grid, dim3(256), 0, s, a);
  else if (cb <= 16)
    hipLaunchKernelGGL((k_quant<16, PUB>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_quant<32, PUB>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// One launch per block of up to 32 rank columns; codes and scales are
// written by the first.  slices = gridDim.y (K-slices of a.kslice channels).
hipError_t launch_quant(const QuantArgs &a0, int slices, hipStream_t s) {
  const bool pub = a0.qx != nullptr;
  const int rows = pub ? a0.M : a0.Mpad;
  dim3 grid((unsigned)ceil_div(rows, 16), (unsigned)slices);
  const int total = a0.r * a0.batch;
  int c0 = 0;
  do {
    QuantArgs a = a0;
    a.c0 = c0;
    a.cb = total - c0 < kRankBlock ? total - c0 : kRankBlock;
    a.write_codes = (c0 == 0);
    hipError_t e = pub ? launch_variant<true>(a, grid, s) : launch_variant<false>(a, grid, s);
    if (e != hipSuccess) return e;
    c0 += kRankBlock;
  } while (c0 < total);
  return hipSuccess;
}

}  // namespace hsq

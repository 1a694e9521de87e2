// quant.hip -- the public quantization pass (hsq_quantize_act): one pass over
// X that smooths it, quantizes it per token in 64-wide groups to symmetric
// int4, and forms the rank-r down projection U = xh * L1 of the smoothed,
// unquantized activations, in the public layout (row-major packed nibbles,
// fp16 scales M x G, U as M x r).  The fused linear uses its own pass in the
// contraction's operand order (quant_tiles.hip); both follow the same
// arithmetic.
//
// Operation (hsq.h formula block): smoothing by a diagonal scale (H-SVDQuant
// explainer, rit.work, section on Hessian deflation), group-64 4-bit
// activations (Deflating the Hessian, Table 1 caption), high-precision
// branch on unquantized inputs (DiRotQ notes, key design 2).
//
// Mapping: one lane per (token, 64-channel group) item.  A workgroup owns
// all ng = K/64 groups (K <= 12288) and a run of tokens, taken `rows` =
// 256/ng tokens at a time (lane t = token t/ng, group t%ng).  A lane loads its group with eight
// 16-byte loads, finds the absmax in registers, computes the fp16 scale and
// its reciprocal once, writes the codes and forms its group's share of U.
// The 1/lambda (exact IEEE division) and, when they fit, the L1 rows
// are staged in LDS once per workgroup, one padded row per group, so that
// lanes of one token read different banks and lanes of different tokens
// read the same words (broadcast).  The first X loads are issued before the
// staging and each row step prefetches the next, so a lane waits for about
// one memory round trip per step.  The U shares of a token are summed
// through LDS in a fixed order.
#include "hsq_internal.h"

namespace hsq {

namespace {

constexpr int kLamStride = kGroup + 4;            // LDS floats per group row of 1/lambda
constexpr size_t kL1StageBytes = 36 * 1024;       // LDS for staged L1 rows
constexpr int kTargetBlocks = 1024;               // workgroups before a launch iterates rows
constexpr int kMaxIters = 16;

constexpr int l1_stride(int nr) { return kGroup * nr + 4; }  // LDS floats per group of L1

int rank_block(int cb) {
  return cb == 0 ? 0 : cb <= 4 ? 4 : cb <= 8 ? 8 : cb <= 12 ? 12 : cb <= 16 ? 16 : 32;
}

size_t stage_bytes(int ng, int nr) { return sizeof(float) * (size_t)ng * l1_stride(nr); }

struct QuantPlan {
  int slices, ng, rows, iters, nr, stage;
  size_t lds;
};

// Staging and LDS size of one rank block of nr columns under plan p.
QuantPlan for_block(QuantPlan p, int nr) {
  p.nr = nr;
  p.stage = nr > 0 && stage_bytes(p.ng, nr) <= kL1StageBytes;
  p.lds = sizeof(float) * ((size_t)(p.ng + 1) * kLamStride + 4 * 256) + (p.stage ? stage_bytes(p.ng, nr) : 0);
  return p;
}

QuantPlan plan(int M, int K, int r) {
  QuantPlan p{};
  p.nr = rank_block(r < kRankBlock ? r : kRankBlock);
  p.slices = 1;
  p.ng = K / kGroup;                               // <= kMaxSliceGroups (entry point checks K)
  p.rows = 256 / p.ng;
  const int row_blocks = ceil_div(M, p.rows);
  int it = row_blocks * p.slices / kTargetBlocks;
  p.iters = it < 1 ? 1 : (it > kMaxIters ? kMaxIters : it);
  return for_block(p, p.nr);
}

template <int NR, bool STAGE>
__global__ __launch_bounds__(256) void k_quant(QuantArgs a, int ng, int rows, int iters) {
  // dynamic LDS: 1/lambda [ng + 1][kLamStride] (last row zero), U shares [4][256],
  // staged L1 [ng][64*NR + 4] (group row: channel-major, NR columns)
  extern __shared__ float lds[];
  float *inv_lam = lds;
  float *upart = inv_lam + (ng + 1) * kLamStride;
  float *l1s = upart + 4 * 256;

  const int tid = threadIdx.x;
  const int gend = a.kend / kGroup;                // groups to write (G or Gp)
  const int gb = blockIdx.y * ng;                  // first group of the slice
  const int gn = min(ng, gend - gb);               // groups in this slice
  const int rl = tid / ng, gi = tid % ng;          // (token, group) of this lane
  const int g = gb + gi;
  const int mrows = a.M;
  const int mbase = blockIdx.x * rows * iters;
  const bool lane_ok = rl < rows && gi < gn;
  const bool g_in = lane_ok && g < a.G;            // else a pad group: zeros

  // ---- loads, oldest first: slice tables, then X (the table stores below
  // wait for the tables only; X stays in flight until the first row step)
  // 1/lambda: thread t loads channels 8(t%8) .. +7 of slice group t/8
  const bool lam_ok = tid < gn * 8 && gb + (tid >> 3) < a.G;
  const v4u lv = *reinterpret_cast<const v4u *>(
      a.lam + (size_t)min(gb + (tid >> 3), a.G - 1) * kGroup + 8 * (tid & 7));
  // L1 (r % 4 == 0): J chunks of four columns per thread, clamped addresses
  constexpr int J = 8;
  const bool vec_l1 = STAGE && (a.r & 3) == 0;
  const int cb4 = a.cb >> 2, n4 = gn * kGroup * cb4;
  auto l1_chunk = [&](int p) __attribute__((always_inline)) {
    const int c4 = cb4 == 1 ? 0 : p % cb4, rest = cb4 == 1 ? p : p / cb4;
    const int k = min((gb + (rest >> 6)) * kGroup + (rest & 63), a.K - 1);
    const int cc = a.c0 + 4 * c4, b = cc / a.r, jj = cc % a.r;
    return reinterpret_cast<const v2u *>(a.L1 + ((size_t)b * a.K + k) * a.r + jj);
  };
  auto l1_store = [&](int p, v2u v) __attribute__((always_inline)) {
    const int c4 = cb4 == 1 ? 0 : p % cb4, rest = cb4 == 1 ? p : p / cb4;
    const int gg = rest >> 6, i = rest & 63;
    *reinterpret_cast<v4f *>(l1s + gg * l1_stride(NR) + i * NR + 4 * c4) =
        gb + gg < a.G ? (v4f){bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16),
                              bf16_to_f32(v.y & 0xFFFFu), bf16_to_f32(v.y >> 16)}
                      : (v4f){0.f, 0.f, 0.f, 0.f};
  };
  // one chunk per channel (four rank columns of one projection): its loads
  // go out with the others; wider blocks are staged in a loop below
  const bool fast_l1 = vec_l1 && cb4 == 1;
  // (issued unconditionally -- a branch here would make the compiler wait
  // for them before the X loads; unused, they read the first L1 chunk)
  v2u l1v[J];
  if (STAGE) {
    const uint16_t *l1 = fast_l1 ? a.L1 + ((size_t)(a.c0 / a.r) * a.K) * a.r + a.c0 % a.r : a.L1;
    const int kstride = fast_l1 ? a.r : 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int rest = min(tid + 256 * j, n4 - 1);
      const int k = min(gb * kGroup + rest, a.K - 1);
      l1v[j] = *reinterpret_cast<const v2u *>(l1 + (size_t)k * kstride);
    }
  }

  v4u raw[8];
  auto load_x = [&](int m) __attribute__((always_inline)) {
    // clamped: rows past M and pad groups read a valid row and are zeroed
    // through the zero 1/lambda row below
    const v4u *src = reinterpret_cast<const v4u *>(a.X + (size_t)min(m, a.M - 1) * a.K +
                                                   (size_t)min(g, a.G - 1) * kGroup);
#pragma unroll
    for (int t = 0; t < 8; ++t) raw[t] = src[t];
  };
  load_x(mbase + rl);

  // ---- slice tables into LDS ----
  auto lam_store = [&](int p, v4u v, bool ok) __attribute__((always_inline)) {
    float f[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      f[2 * h] = ok ? 1.0f / f16_to_f32((uint16_t)(v[h] & 0xFFFFu)) : 0.0f;
      f[2 * h + 1] = ok ? 1.0f / f16_to_f32((uint16_t)(v[h] >> 16)) : 0.0f;
    }
    v4f *dst = reinterpret_cast<v4f *>(inv_lam + (p >> 3) * kLamStride + 8 * (p & 7));
    dst[0] = (v4f){f[0], f[1], f[2], f[3]};
    dst[1] = (v4f){f[4], f[5], f[6], f[7]};
  };
  if (tid < gn * 8) lam_store(tid, lv, lam_ok);
  for (int p = tid + 256; p < gn * 8; p += 256) {  // more than 32 groups
    const bool ok = gb + (p >> 3) < a.G;
    const v4u v = *reinterpret_cast<const v4u *>(
        a.lam + (size_t)min(gb + (p >> 3), a.G - 1) * kGroup + 8 * (p & 7));
    lam_store(p, v, ok);
  }
  if (tid < kGroup) inv_lam[ng * kLamStride + tid] = 0.0f;  // zero row: rows past M
  if (fast_l1) {
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (tid + 256 * j < n4) l1_store(tid + 256 * j, l1v[j]);
    for (int p = tid + 256 * J; p < n4; p += 256) l1_store(p, *l1_chunk(p));
  } else if (vec_l1) {
    for (int p = tid; p < n4; p += 256) l1_store(p, *l1_chunk(p));
  } else if (STAGE) {
    // odd ranks: one column per element
    for (int p = tid; p < gn * kGroup * a.cb; p += 256) {
      const int c = p % a.cb, rest = p / a.cb, gg = rest >> 6, i = rest & 63;
      const int k = min((gb + gg) * kGroup + i, a.K - 1);
      const int cc = a.c0 + c, b = cc / a.r, jj = cc % a.r;
      l1s[gg * l1_stride(NR) + i * NR + c] =
          gb + gg < a.G ? bf16_to_f32(a.L1[((size_t)b * a.K + k) * a.r + jj]) : 0.0f;
    }
  }
  __syncthreads();

  const float *l1_row = l1s + gi * l1_stride(NR);

  for (int it = 0; it < iters; ++it) {
    const int mb = mbase + it * rows;
    if (mb >= mrows) break;                        // uniform over the workgroup
    const int m = mb + rl;
    const bool live = lane_ok && m < mrows;
    const bool in = g_in && m < a.M;
    const float *lam_row = inv_lam + (in ? gi : ng) * kLamStride;

    float xh[kGroup];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const v4f l0 = *reinterpret_cast<const v4f *>(lam_row + 8 * t);
      const v4f l1 = *reinterpret_cast<const v4f *>(lam_row + 8 * t + 4);
      xh[8 * t + 0] = bf16_to_f32(raw[t].x & 0xFFFFu) * l0.x;
      xh[8 * t + 1] = bf16_to_f32(raw[t].x >> 16) * l0.y;
      xh[8 * t + 2] = bf16_to_f32(raw[t].y & 0xFFFFu) * l0.z;
      xh[8 * t + 3] = bf16_to_f32(raw[t].y >> 16) * l0.w;
      xh[8 * t + 4] = bf16_to_f32(raw[t].z & 0xFFFFu) * l1.x;
      xh[8 * t + 5] = bf16_to_f32(raw[t].z >> 16) * l1.y;
      xh[8 * t + 6] = bf16_to_f32(raw[t].w & 0xFFFFu) * l1.z;
      xh[8 * t + 7] = bf16_to_f32(raw[t].w >> 16) * l1.w;
    }
    if (it + 1 < iters) load_x(m + rows);          // next row step, in flight meanwhile

    if (live && a.write_codes) {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < kGroup; ++i) amax = fmaxf(amax, fabsf(xh[i]));
      uint16_t s16 = 0;
      if (amax != 0.0f) {
        s16 = f32_to_f16(amax / 7.0f);
        if (s16 == 0x7C00u) s16 = 0x7BFFu;         // saturate at 65504
      }
      const float s = f16_to_f32(s16);
      const float inv_s = (s16 != 0) ? 1.0f / s : 0.0f;
      // code = clamp(rint(fl32(xh / s)), -8, 7): adding 1.5 * 2^23 rounds the
      // fp32 quotient to an integer (ties to even) in the low mantissa bits;
      // the clamp works on those bits (a quotient beyond +-2^22 lands outside
      // the clamp window on the right side).  The low byte of the clamped
      // bits is the two's-complement code.
      int c[kGroup];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const float t = xh[i] * inv_s;
        const int b = __float_as_int(t + kMagic);
        c[i] = min(max(b, kMagicBits - 8), kMagicBits + 7);
      }
      if (in) {
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t v = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) v |= (uint32_t)(c[8 * j + e] & 0xF) << (4 * e);
          w[j] = v;
        }
        v4u *dst = reinterpret_cast<v4u *>(a.qx + (size_t)m * (a.K / 2) + (size_t)g * 32);
        dst[0] = (v4u){w[0], w[1], w[2], w[3]};
        dst[1] = (v4u){w[4], w[5], w[6], w[7]};
        a.sx[(size_t)m * a.G + g] = s16;
      }
    }

    // ---- U: four rank columns at a time, summed over the slice's groups ----
    if (NR > 0) {
#pragma unroll
      for (int c4 = 0; c4 < NR; c4 += 4) {
        if (c4 >= a.cb) break;                     // uniform
        if (STAGE) {
          float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
          if (in) {
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
              const v4f l = *reinterpret_cast<const v4f *>(l1_row + i * NR + c4);
              s0 = __builtin_fmaf(xh[i], l.x, s0);
              s1 = __builtin_fmaf(xh[i], l.y, s1);
              s2 = __builtin_fmaf(xh[i], l.z, s2);
              s3 = __builtin_fmaf(xh[i], l.w, s3);
            }
          }
          upart[0 * 256 + tid] = s0;
          upart[1 * 256 + tid] = s1;
          upart[2 * 256 + tid] = s2;
          upart[3 * 256 + tid] = s3;
        } else {
          // L1 rows from the cache, one column at a time, 16 channels in flight
#pragma unroll 1
          for (int e = 0; e < 4; ++e) {
            float acc = 0.0f;
            if (in && c4 + e < a.cb) {
              const int cc = a.c0 + c4 + e, b = cc / a.r, j = cc % a.r;
              const uint16_t *l1 = a.L1 + ((size_t)b * a.K + (size_t)g * kGroup) * a.r + j;
#pragma unroll
              for (int i0 = 0; i0 < kGroup; i0 += 16) {
#pragma unroll
                for (int i = i0; i < i0 + 16; ++i) acc = __builtin_fmaf(xh[i], bf16_to_f32(l1[(size_t)i * a.r]), acc);
                asm volatile("" : "+v"(acc) : : "memory");
              }
            }
            upart[e * 256 + tid] = acc;
          }
        }
        __syncthreads();
        const int cw = min(4, a.cb - c4);
        for (int p = tid; p < rows * cw; p += 256) {   // rows * cw > 256 when ng < 4
          const int r0 = p % rows, e = p / rows;
          const int mm = mb + r0;
          if (mm < mrows) {
            const float *src = upart + e * 256 + r0 * ng;
            float s = 0.0f;
            for (int q = 0; q < gn; ++q) s += src[q];
            a.u_pub[(size_t)mm * a.r + a.c0 + c4 + e] = s;
          }
        }
        __syncthreads();
      }
    }
  }
}

template <bool STAGE>
hipError_t launch_nr(const QuantArgs &a, const QuantPlan &p, int nr, dim3 grid, hipStream_t s) {
  switch (nr) {
    case 0: hipLaunchKernelGGL((k_quant<0, false>), grid, dim3(256), p.lds, s, a, p.ng, p.rows, p.iters); break;
    case 4: hipLaunchKernelGGL((k_quant<4, STAGE>), grid, dim3(256), p.lds, s, a, p.ng, p.rows, p.iters); break;
    case 8: hipLaunchKernelGGL((k_quant<8, STAGE>), grid, dim3(256), p.lds, s, a, p.ng, p.rows, p.iters); break;
    case 12: hipLaunchKernelGGL((k_quant<12, STAGE>), grid, dim3(256), p.lds, s, a, p.ng, p.rows, p.iters); break;
    case 16: hipLaunchKernelGGL((k_quant<16, STAGE>), grid, dim3(256), p.lds, s, a, p.ng, p.rows, p.iters); break;
    default: hipLaunchKernelGGL((k_quant<32, STAGE>), grid, dim3(256), p.lds, s, a, p.ng, p.rows, p.iters); break;
  }
  return hipGetLastError();
}

}  // namespace

// One launch per block of up to 32 rank columns; codes and scales are
// written by the first.
hipError_t launch_quant_act(const QuantArgs &a0, hipStream_t s) {
  const QuantPlan p = plan(a0.M, a0.K, a0.r);
  if (p.ng < 1 || p.ng > kMaxSliceGroups) return hipErrorInvalidValue;
  dim3 grid((unsigned)ceil_div(a0.M, p.rows * p.iters), 1u);
  const int total = a0.r;
  int c0 = 0;
  do {
    QuantArgs a = a0;
    a.c0 = c0;
    a.cb = total - c0 < kRankBlock ? total - c0 : kRankBlock;
    a.write_codes = (c0 == 0);
    // a later rank block may be narrower than the first: same grid, its own
    // template and LDS size
    const int nr = rank_block(a.cb);
    const QuantPlan q = for_block(p, nr);
    const hipError_t e = q.stage ? launch_nr<true>(a, q, nr, grid, s) : launch_nr<false>(a, q, nr, grid, s);
    if (e != hipSuccess) return e;
    c0 += kRankBlock;
  } while (c0 < total);
  return hipSuccess;
}

}  // namespace hsq

// quant_tiles.hip -- K1 of the fused linear: one pass over X that smooths it,
// quantizes it per token in 64-wide groups to symmetric int4 (written as int8
// codes in the contraction's MFMA operand order, with fp16 scales), and
// accumulates the rank-r down projection U = xh * L1 of the smoothed,
// unquantized activations.
//
// Operation (hsq.h formula block): smoothing by a diagonal scale (H-SVDQuant
// explainer, rit.work, section on Hessian deflation), group-64 4-bit
// activations (Deflating the Hessian, Table 1 caption), high-precision
// branch on unquantized inputs (DiRotQ notes, key design 2).
//
// Mapping: a workgroup owns one 16-row tile and a K-slice of scale groups
// (64 channels, or 128 -- two 64-channel blocks -- for group-128, Deflating
// the Hessian, Table 3 caption); its waves take the slice's groups
// round-robin.  For a 64-channel block, lane l holds row l%16 and channels
// 16*(l/16) .. +15 -- exactly lane l's 16-byte slot of the int8 MFMA operand
// block (row tile, block) -- so X arrives as two 16-byte loads per lane and
// block (64 contiguous bytes per row and load) and the codes leave as one
// contiguous 1 KB store per wave and block.  The group absmax is a 4-lane
// exchange (lanes l, l^16, l^32, l^48 hold the row's four channel blocks).
// 1/lambda (exact IEEE division, once per channel) and L1 (fp32) of the
// slice are staged in LDS, padded so that the four channel blocks of a
// group fall in different banks.  Each lane keeps its row's share of U over
// all the groups it visits; the block sums the shares of its waves and
// channel blocks in a fixed order and writes one U partial per K-slice,
// which the contraction kernels sum in slice order.  Rows past M read zero
// through the range-checked buffer loads and a pad group has zero 1/lambda,
// so both produce zero codes, scales and U without a branch.
#include "hsq_internal.h"

#include <type_traits>

namespace hsq {

namespace {

constexpr int kRankPass = 16;              // rank columns one pass accumulates
constexpr size_t kSliceLdsBytes = 40 * 1024;  // staged 1/lambda + L1 per workgroup
constexpr int kTargetWaves = 2048;         // waves a launch aims for (8 per CU)
constexpr int kOneUnitWaves = 20 * 256;    // one unit per wave up to this many waves
constexpr int kLamKq = 16 + 4;             // LDS floats per (group, channel block) of 1/lambda

constexpr int kqs(int nr) { return 16 * nr + 4; }  // LDS floats per (group, channel block) of L1

int pass_width(int cb) { return cb == 0 ? 0 : cb <= 4 ? 4 : cb <= 8 ? 8 : cb <= 12 ? 12 : 16; }

struct TilePlan {
  int slices, gpb, waves, nr;
};

// the U shares reuse the tables' LDS once every wave has left the loop;
// gpb units of bpg blocks each
size_t plan_lds(int gpb, int bpg, int nr, int waves) {
  const size_t tables = (size_t)gpb * bpg * 4 * (kLamKq + kqs(nr)), shares = (size_t)waves * 64 * nr;
  return sizeof(float) * (tables > shares ? tables : shares);
}

// Work units: scale groups of bpg 64-channel blocks (every padded block for
// group 64, every 128-channel group for group 128).  K-slices: enough for
// the staged tables to fit kSliceLdsBytes and, up to kMaxUSlices, for about
// kTargetWaves waves of 4; few row tiles get wider workgroups (up to 16
// waves, at most one per unit of the slice).
TilePlan tile_plan(int M, int K, int r, int batch, int group) {
  TilePlan p{};
  const int MT = ceil_div(M, kTile), Gp = scale_groups_stored(K, group), bpg = group / kGroup;
  const int total = r * batch;
  p.nr = pass_width(total < kRankPass ? total : kRankPass);
  const size_t per_group = sizeof(float) * bpg * (4 * kLamKq + 4 * kqs(p.nr));
  int fit = (int)(kSliceLdsBytes / per_group);
  if (fit < 1) fit = 1;
  int S = ceil_div(Gp, fit);
  const int want = ceil_div(kTargetWaves, MT * 4);
  const int more = want < kMaxUSlices ? want : kMaxUSlices;
  if (more > S) S = more;
  // few tokens: the pass is a chain of latencies, so no wave takes a second
  // unit -- at most 16 units per slice, one per wave of a 16-wave workgroup
  // (Qwen3 down at 16 tokens: 8 slices of 24 units, 17.0 us per layer, ->
  // 12 slices of 16; the skinny contraction prefetches up to 16 U slices)
  if (M <= kSkinnyMaxM && S < ceil_div(Gp, 16)) S = ceil_div(Gp, 16);
  if (S > Gp) S = Gp;
  p.gpb = ceil_div(Gp, S);
  p.slices = ceil_div(Gp, p.gpb);
  // waves per workgroup: 8 when each gets two or more groups of the slice
  // (more loads in flight per CU), else 4; one unit per wave (every load of
  // the slice in flight at once) when the launch is small or still fits one
  // round of the chip at that width (at most 20 waves per CU: pixart's 512
  // workgroups of 9 waves, 7.1 -> 6.2 us; wider launches lose a round)
  p.waves = p.gpb >= 16 ? 8 : 4;
  if ((long long)MT * p.slices * 4 < kTargetWaves / 2 || (long long)MT * p.slices * p.gpb <= kOneUnitWaves)
    p.waves = p.gpb < 4 ? 4 : (p.gpb > 16 ? 16 : p.gpb);
  return p;
}

// code modes: rank pass only, symmetric codes, asymmetric codes
constexpr int kNoCodes = 0, kSymCodes = 1, kAsymCodes = 2;

template <int NR, int CM, int BPG, bool ONE>
__global__ __launch_bounds__(1024) void k_quant_tiles(QuantArgs a, int gpb) {
  // dynamic LDS: 1/lambda [gpb*BPG][4][kLamKq], L1 [gpb*BPG][4][kqs(NR)]
  // (per 64-block and channel block: 16 channels x NR columns); after the
  // loop, U shares [waves][NR][64]
  extern __shared__ float lds[];
  const int MT = a.Mpad / kTile;
  if ((int)blockIdx.x >= MT) {
    // workgroups past the row tiles write the contraction's weight-scale
    // pairs (first pass only), grid-strided over the table
    const size_t total8 = (size_t)a.batch * a.swr * (a.swnpad / 8);
    const size_t px = gridDim.x - (unsigned)MT, step = px * gridDim.y * blockDim.x;
    for (size_t i = ((size_t)(blockIdx.x - MT) + px * blockIdx.y) * blockDim.x + threadIdx.x; i < total8; i += step)
      sw_pair_item(a.sw, a.swG, a.swN, a.swr, a.swnpad, i, a.swp);
    return;
  }
  float *ilam = lds;
  float *l1s = ilam + gpb * BPG * 4 * kLamKq;
  float *upart = lds;

  const int nthr = (int)blockDim.x, W = nthr >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mt = blockIdx.x;
  const int nunits = a.SG;                    // scale groups per row tile (the units)
  const int gs = blockIdx.y * gpb;
  const int ge = min(gs + gpb, nunits), ngb = ge - gs;
  const int nblk = ngb * BPG;                 // 64-blocks of the slice
  const int row = lane & 15, kq = lane >> 4;
  const int m = mt * kTile + row;

  // X through a resource of exactly M*K bf16 (M*K < 2^31): rows past M get
  // the offset at its end and read zero (the range check covers the lane
  // offset); the block offset is scalar and clamped to the last real block
  // (a pad block reads that one and zeroes it through its zero 1/lambda)
  const uint32_t xbytes = (uint32_t)((size_t)a.M * a.K * 2);
  const __amdgpu_buffer_rsrc_t rs_x = buffer_rsrc(a.X, xbytes);
  const uint32_t offx = m < a.M ? ((uint32_t)m * (uint32_t)a.K + 16u * kq) * 2u : xbytes;
  // the unit's BPG blocks, two 16-byte loads each
  // (the block index is uniform; readfirstlane lets the compiler see it, or
  // it wraps each load in a loop over the lanes' values)
  auto load_x = [&](int g, v4u (&x)[2 * BPG]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < BPG; ++b) {
      const int bc = __builtin_amdgcn_readfirstlane(min(g * BPG + b, a.G - 1));
      x[2 * b] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, offx, bc * 128, 0);
      x[2 * b + 1] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, offx, bc * 128 + 16, 0);
    }
  };
  // the wave's units are g0, g0 + W, ...; the first loads during the table
  // staging.  ONE (at most one unit per wave): a wave past the slice loads
  // with the out-of-range lane offset (zero, no memory traffic), and no
  // further load follows.  Otherwise the next unit is in flight while one
  // is processed.
  const int g0 = gs + wave;
  v4u x[2 * BPG];
  if constexpr (ONE) {
    const uint32_t off = g0 < ge ? offx : xbytes;
#pragma unroll
    for (int b = 0; b < BPG; ++b) {
      const int bc = min(g0 * BPG + b, a.G - 1);
      x[2 * b] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, off, bc * 128, 0);
      x[2 * b + 1] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, off, bc * 128 + 16, 0);
    }
  } else {
    load_x(min(g0, ge - 1), x);               // in flight during the staging (unused past the slice)
  }

  // ---- slice tables: 1/lambda, 8 channels per item ----
  const int bs = gs * BPG;                    // first 64-block of the slice
  for (int p = tid; p < nblk * 8; p += nthr) {
    const int bl = p >> 3, c = 8 * (p & 7);
    const bool real = bs + bl < a.G;
    const v4u lv = *reinterpret_cast<const v4u *>(a.lam + (size_t)min(bs + bl, a.G - 1) * kGroup + c);
    float f[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      f[2 * h] = real ? 1.0f / f16_to_f32((uint16_t)(lv[h] & 0xFFFFu)) : 0.0f;
      f[2 * h + 1] = real ? 1.0f / f16_to_f32((uint16_t)(lv[h] >> 16)) : 0.0f;
    }
    v4f *dst = reinterpret_cast<v4f *>(ilam + (bl * 4 + (c >> 4)) * kLamKq + (c & 15));
    dst[0] = (v4f){f[0], f[1], f[2], f[3]};
    dst[1] = (v4f){f[4], f[5], f[6], f[7]};
  }
  // ---- L1 columns [c0, c0 + cb) of the batch*r columns, zero past cb ----
  if constexpr (NR > 0) {
    if ((a.r & 3) == 0) {
      // four columns of one projection per item (cb and c0 are multiples of 4)
      constexpr int Q = NR / 4;
      for (int p = tid; p < nblk * kGroup * Q; p += nthr) {
        const int q4 = p % Q, chl = p / Q, bl = chl >> 6, c = chl & 63;
        const int gg = bs + bl, jj = 4 * q4;
        v4f v = {0.f, 0.f, 0.f, 0.f};
        if (gg < a.G && jj < a.cb) {
          const int cc = a.c0 + jj, b = cc / a.r, j = cc % a.r;
          const v2u w = *reinterpret_cast<const v2u *>(a.L1 + ((size_t)b * a.K + (size_t)gg * kGroup + c) * a.r + j);
          v = (v4f){bf16_to_f32(w.x & 0xFFFFu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xFFFFu),
                    bf16_to_f32(w.y >> 16)};
        }
        *reinterpret_cast<v4f *>(l1s + (bl * 4 + (c >> 4)) * kqs(NR) + (c & 15) * NR + jj) = v;
      }
    } else {
      for (int p = tid; p < nblk * kGroup * NR; p += nthr) {
        const int jj = p % NR, chl = p / NR, bl = chl >> 6, c = chl & 63;
        const int gg = bs + bl;
        float v = 0.0f;
        if (gg < a.G && jj < a.cb) {
          const int cc = a.c0 + jj, b = cc / a.r, j = cc % a.r;
          v = bf16_to_f32(a.L1[((size_t)b * a.K + (size_t)gg * kGroup + c) * a.r + j]);
        }
        l1s[(bl * 4 + (c >> 4)) * kqs(NR) + (c & 15) * NR + jj] = v;
      }
    }
  }
  __syncthreads();

  float u[NR > 0 ? NR : 1];
#pragma unroll
  for (int j = 0; j < (NR > 0 ? NR : 1); ++j) u[j] = 0.0f;

  auto unit = [&](int g, const v4u (&x)[2 * BPG]) __attribute__((always_inline)) {
    const int gl = g - gs;
    float xh[16 * BPG];
#pragma unroll
    for (int b = 0; b < BPG; ++b) {
      const v4f *il = reinterpret_cast<const v4f *>(ilam + ((gl * BPG + b) * 4 + kq) * kLamKq);
      const v4f l0 = il[0], l1 = il[1], l2 = il[2], l3 = il[3];
      const v4u x0 = x[2 * b], x1 = x[2 * b + 1];
      float *h = xh + 16 * b;
      h[0] = bf16_to_f32(x0.x & 0xFFFFu) * l0.x;
      h[1] = bf16_to_f32(x0.x >> 16) * l0.y;
      h[2] = bf16_to_f32(x0.y & 0xFFFFu) * l0.z;
      h[3] = bf16_to_f32(x0.y >> 16) * l0.w;
      h[4] = bf16_to_f32(x0.z & 0xFFFFu) * l1.x;
      h[5] = bf16_to_f32(x0.z >> 16) * l1.y;
      h[6] = bf16_to_f32(x0.w & 0xFFFFu) * l1.z;
      h[7] = bf16_to_f32(x0.w >> 16) * l1.w;
      h[8] = bf16_to_f32(x1.x & 0xFFFFu) * l2.x;
      h[9] = bf16_to_f32(x1.x >> 16) * l2.y;
      h[10] = bf16_to_f32(x1.y & 0xFFFFu) * l2.z;
      h[11] = bf16_to_f32(x1.y >> 16) * l2.w;
      h[12] = bf16_to_f32(x1.z & 0xFFFFu) * l3.x;
      h[13] = bf16_to_f32(x1.z >> 16) * l3.y;
      h[14] = bf16_to_f32(x1.w & 0xFFFFu) * l3.z;
      h[15] = bf16_to_f32(x1.w >> 16) * l3.w;
    }

    if constexpr (CM != kNoCodes) {
      uint16_t s16 = 0;
      int zq = 0;                                 // zero point (asymmetric codes)
      float gmin = 0.0f;                          // group minimum, widened to 0 (asymmetric)
      if constexpr (CM == kSymCodes) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16 * BPG; ++i) amax = fmaxf(amax, fabsf(xh[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        if (amax != 0.0f) {
          s16 = f32_to_f16(amax / 7.0f);
          if (s16 == 0x7C00u) s16 = 0x7BFFu;      // saturate at 65504
        }
      } else {
        // asymmetric: the group's range widened to contain 0, 16 levels
        float gmax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16 * BPG; ++i) {
          gmin = fminf(gmin, xh[i]);
          gmax = fmaxf(gmax, xh[i]);
        }
        gmin = fminf(gmin, __shfl_xor(gmin, 16));
        gmin = fminf(gmin, __shfl_xor(gmin, 32));
        gmax = fmaxf(gmax, __shfl_xor(gmax, 16));
        gmax = fmaxf(gmax, __shfl_xor(gmax, 32));
        const float range = gmax - gmin;
        if (range != 0.0f) {
          s16 = f32_to_f16(range / 15.0f);
          if (s16 == 0x7C00u) s16 = 0x7BFFu;      // saturate at 65504
        }
      }
      const float s = f16_to_f32(s16);
      const float inv_s = (s16 != 0) ? 1.0f / s : 0.0f;
      // code = clamp(rint(fl32(xh / s)), -8, 7): adding 1.5 * 2^23 rounds the
      // fp32 quotient to an integer (ties to even) in the low mantissa bits;
      // the clamp works on those bits (a quotient beyond +-2^22 lands outside
      // the clamp window on the right side).  The low byte of the clamped
      // bits is the two's-complement code.  Asymmetric: zero point z =
      // clamp(rint(fl32(-gmin / s)), 0, 15), code q = clamp(rint(fl32(xh / s))
      // + z, 0, 15), and the operand holds q - z (in [-15, 15]).
      if constexpr (CM == kAsymCodes) zq = min(max(__float_as_int(-gmin * inv_s + kMagic) - kMagicBits, 0), 15);
#pragma unroll
      for (int b = 0; b < BPG; ++b) {
        int c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = __float_as_int(xh[16 * b + i] * inv_s + kMagic);
          if constexpr (CM == kSymCodes)
            c[i] = min(max(v, kMagicBits - 8), kMagicBits + 7);
          else
            c[i] = min(max(v + zq, kMagicBits), kMagicBits + 15) - zq;
        }
        v4u w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = __builtin_amdgcn_perm((uint32_t)c[4 * j + 1], (uint32_t)c[4 * j], 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm((uint32_t)c[4 * j + 3], (uint32_t)c[4 * j + 2], 0x0c0c0400u);
          w[j] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        const size_t blk = (size_t)mt * a.Gp + (size_t)g * BPG + b;
        *reinterpret_cast<v4u *>(a.qa + blk * 1024 + (size_t)lane * 16) = w;
      }
      if (kq == 0) a.sxs[((size_t)mt * a.SG + g) * 16 + row] = s16;
    }

    if constexpr (NR > 0) {
#pragma unroll
      for (int b = 0; b < BPG; ++b) {
        const float *lr = l1s + ((gl * BPG + b) * 4 + kq) * kqs(NR);
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
          for (int j4 = 0; j4 < NR; j4 += 4) {
            const v4f l = *reinterpret_cast<const v4f *>(lr + i * NR + j4);
            u[j4 + 0] = __builtin_fmaf(xh[16 * b + i], l.x, u[j4 + 0]);
            u[j4 + 1] = __builtin_fmaf(xh[16 * b + i], l.y, u[j4 + 1]);
            u[j4 + 2] = __builtin_fmaf(xh[16 * b + i], l.z, u[j4 + 2]);
            u[j4 + 3] = __builtin_fmaf(xh[16 * b + i], l.w, u[j4 + 3]);
          }
      }
    }
  };
  if constexpr (ONE) {
    if (g0 < ge) unit(g0, x);
  } else {
    for (int g = g0; g < ge; g += W) {
      // next unit of this wave in flight (past the slice: a clamped, unused
      // load, so that the code stays straight-line and the waits exact)
      v4u nx[2 * BPG];
      load_x(min(g + W, ge - 1), nx);
      unit(g, x);
#pragma unroll
      for (int t = 0; t < 2 * BPG; ++t) x[t] = nx[t];
    }
  }

  // ---- U of the slice: shares of (wave, channel block) summed in that
  // order for each (row, column) ----
  if constexpr (NR > 0) {
    __syncthreads();                            // tables no longer read
#pragma unroll
    for (int j = 0; j < NR; ++j) upart[(wave * NR + j) * 64 + lane] = u[j];
    __syncthreads();
    for (int it = tid; it < kTile * NR; it += nthr) {
      const int rr = it & 15, j = it >> 4;
      float s = 0.0f;
      for (int w = 0; w < W; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) s += upart[(w * NR + j) * 64 + q * 16 + rr];
      if (j < a.cb) a.uw[((size_t)blockIdx.y * a.ucols + a.c0 + j) * a.Mpad + mt * kTile + rr] = s;
    }
  }
}

template <int NR, int BPG>
hipError_t launch_pass(const QuantArgs &a, const TilePlan &p, int cm, hipStream_t s) {
  // extra columns of workgroups for the weight-scale pairs: one item of 8
  // pairs per thread (a loop of several per thread outlasts the pass at
  // small M)
  int px = 0;
  if (a.swp != nullptr) {
    const size_t total8 = (size_t)a.batch * a.swr * (a.swnpad / 8);
    const size_t per = (size_t)64 * p.waves * p.slices;
    px = (int)((total8 + per - 1) / per);
  }
  const dim3 grid((unsigned)(a.Mpad / kTile + px), (unsigned)p.slices);
  const dim3 block((unsigned)(64 * p.waves));
  const size_t lds = plan_lds(p.gpb, BPG, NR, p.waves);
  // at most one unit per wave (the plan's one-unit-per-wave widths): no
  // look-ahead load.  Measured: Qwen3 down at 16 tokens 5.8 -> 5.5 us, pixart
  // 8.9 -> 8.5 us per pass.  Loading every unit of a wave before the staging
  // instead of one ahead was slower on the large layers (FLUX.1 MLP 27.1 ->
  // 30.3 us per pass, SANA QKV 17.2 -> 18.6 us) and is not used.
  auto go = [&](auto onec) {
    constexpr bool O = decltype(onec)::value;
    if (cm == kSymCodes)
      hipLaunchKernelGGL((k_quant_tiles<NR, kSymCodes, BPG, O>), grid, block, lds, s, a, p.gpb);
    else if (cm == kAsymCodes)
      hipLaunchKernelGGL((k_quant_tiles<NR, kAsymCodes, BPG, O>), grid, block, lds, s, a, p.gpb);
    else
      hipLaunchKernelGGL((k_quant_tiles<NR, kNoCodes, BPG, O>), grid, block, lds, s, a, p.gpb);
  };
  if (p.gpb <= p.waves) go(std::true_type{});
  else go(std::false_type{});
  return hipGetLastError();
}

template <int BPG>
hipError_t launch_width(const QuantArgs &a, const TilePlan &p, int cm, hipStream_t s) {
  switch (pass_width(a.cb)) {
    case 0: return launch_pass<0, BPG>(a, p, cm, s);
    case 4: return launch_pass<4, BPG>(a, p, cm, s);
    case 8: return launch_pass<8, BPG>(a, p, cm, s);
    case 12: return launch_pass<12, BPG>(a, p, cm, s);
    default: return launch_pass<16, BPG>(a, p, cm, s);
  }
}

}  // namespace

int quant_slices(int M, int K, int r, int batch, int group) {
  return tile_plan(M, K, r, batch, group).slices;
}

// One launch per pass of up to 16 rank columns; the first also writes codes
// and scales.  Every pass uses the first pass's grid (same K-slices, so the
// U partials line up).
hipError_t launch_quant_tiles(const QuantArgs &a0, hipStream_t s) {
  const int group = a0.bpg * kGroup;
  const TilePlan p = tile_plan(a0.M, a0.K, a0.r, a0.batch, group);
  if (plan_lds(p.gpb, a0.bpg, p.nr, p.waves) > 64 * 1024) return hipErrorInvalidValue;
  const int total = a0.r * a0.batch;
  int c0 = 0;
  do {
    QuantArgs a = a0;
    a.c0 = c0;
    a.cb = total - c0 < kRankPass ? total - c0 : kRankPass;
    const int cm = c0 != 0 ? kNoCodes : a.asym ? kAsymCodes : kSymCodes;
    if (c0 != 0) a.swp = nullptr;
    const hipError_t e = a.bpg == 2 ? launch_width<2>(a, p, cm, s) : launch_width<1>(a, p, cm, s);
    if (e != hipSuccess) return e;
    c0 += kRankPass;
  } while (c0 < total);
  return hipSuccess;
}

}  // namespace hsq

// gemm_skinny.hip -- K2 (SKINNY): the residual contraction for small token
// counts (M <= 64), where the layer is bound by streaming the packed weights
// from HBM (K*N/2 bytes for 2*M*N*K operations).
//
// Same arithmetic as the tiled kernel (hsq.h formula block; one 16x16x64
// int8 MFMA per group and output tile, magic-constant accumulator, two FMAs
// per element and group).  Mapping: a workgroup owns CT adjacent 16-column
// tiles of one projection; its W waves split the K groups into runs of P
// group pairs (P, CT fixed at compile time).  For a run, a wave issues the
// loads of all P x CT weight blocks (1 KB each, 16 bytes per lane, straight
// from HBM into registers) together with the run's activation codes and
// scales (shared by the CT tiles, from the cache) before it computes
// anything, so the whole weight stream of the chip is in flight at once.
// The W partial tiles meet in LDS after one barrier; each thread then sums
// one output over the waves in wave order (deterministic) and adds U * L2
// and the bias -- no split-K buffer, one launch.
#include "hsq_internal.h"

namespace hsq {

namespace {

constexpr uint32_t kNibMask = 0xF0F0F0F0u;
// cache policy of the weight stream (read once): non-temporal
constexpr int kStreamLoad = 2;
// waves per workgroup: up to 16 for one or two row tiles, 8 for more (whose
// registers need the larger per-wave budget)
constexpr int max_waves(int mt) { return mt <= 2 ? 16 : 8; }

template <int MT, int P, int CT, bool DUMP, int BPG>
__global__ __launch_bounds__(64 * max_waves(MT)) void k_gemm_skinny(GemmArgs a, int W) {
  // a block pair of the packed residual is two 64-channel groups (BPG = 1)
  // or one 128-channel group (BPG = 2: its two MFMAs accumulate in int32,
  // then one rescale)
  constexpr int NS = BPG == 1 ? 2 : 1;              // scale groups per block pair
  // dynamic LDS: partial tiles [W][CT][MT][4][64], then U [r][16*MT]
  // (slices summed), L2 [r][16*CT], bias [16*CT]
  extern __shared__ float red[];
  float *eu = red + W * CT * MT * 4 * 64;
  float *el2 = eu + a.r * MT * 16;
  float *eb = el2 + a.r * 16 * CT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = (a.N + 15) / 16;
  const int nt0 = (blockIdx.x + (DUMP ? a.n0 / (16 * CT) : 0)) * CT;   // first column tile
  const int proj = blockIdx.y;
  const int GP = a.Gp / 2, G = a.G;
  const int colq = lane & 15, rowq = 4 * (lane >> 4);
  const v4i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};

  const __amdgpu_buffer_rsrc_t rs_w =
      buffer_rsrc(a.w + (size_t)proj * a.w_stride, (uint32_t)NT * GP * 1024);
  const __amdgpu_buffer_rsrc_t rs_a = buffer_rsrc(a.qa, (uint32_t)MT * a.Gp * 1024);
  const __amdgpu_buffer_rsrc_t rs_x = buffer_rsrc(a.sxs, (uint32_t)MT * a.SG * 32);
  const __amdgpu_buffer_rsrc_t rs_s =
      buffer_rsrc(DUMP ? nullptr : a.sw + (size_t)proj * G * a.N, DUMP ? 0u : (uint32_t)G * a.N * 2);
  uint32_t offw[CT], offsw[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int nt = min(nt0 + c, NT - 1);            // past the last tile: clamped, not stored
    offw[c] = ((uint32_t)nt * GP * 64 + lane) * 16;
    offsw[c] = (uint32_t)min(nt * 16 + colq, a.N - 1) * 2;
  }

  float acc[CT][MT][4];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[c][i][q] = 0.0f;

  const int EUN = a.r * MT * 16, ELN = a.r * 16 * CT, nthr = W * 64;

  // activation codes / scales of one group pair, raw weight scales of its
  // CT column tiles
  struct Act {
    v4i av[MT][2];
    v4h sx[MT][NS];
    _Float16 sw[CT][NS];
  };
  auto load_act = [&](int gp, Act &t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        t.av[i][h] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(rs_a, (uint32_t)(i * a.Gp * 64 + lane) * 16,
                                                       (2 * gp + h) * 1024, 0));
    if (!DUMP) {
      // scale group sg of the pair: 2gp + h (group 64) or gp (group 128).
      // A pad group (sg = G) reads group G-1: its codes are zero, so it adds
      // fma(1.5*2^23, sw, -1.5*2^23*sw) = 0 exactly whatever sw is
#pragma unroll
      for (int h = 0; h < NS; ++h) {
        const int sg = NS * gp + h;
#pragma unroll
        for (int i = 0; i < MT; ++i)
          t.sx[i][h] = __builtin_bit_cast(
              v4h, __builtin_amdgcn_raw_buffer_load_b64(rs_x, (uint32_t)(i * a.SG * 16 + rowq) * 2, sg * 32, 0));
#pragma unroll
        for (int c = 0; c < CT; ++c)
          t.sw[c][h] = __builtin_bit_cast(
              _Float16, __builtin_amdgcn_raw_buffer_load_b16(rs_s, offsw[c], min(sg, G - 1) * a.N * 2, 0));
      }
    }
  };

  // runs of P group pairs: wave w takes pairs [c0, c0 + P) for c0 = P*w,
  // P*(w + W), ...
  for (int c0 = wave * P; c0 < GP; c0 += W * P) {
    const int pn = min(P, GP - c0);               // pairs in this run (uniform)
    v4u wv[P][CT];
    Act t[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int gp = min(c0 + p, GP - 1);
      load_act(gp, t[p]);
#pragma unroll
      for (int c = 0; c < CT; ++c)
        wv[p][c] = __builtin_amdgcn_raw_buffer_load_b128(rs_w, offw[c], gp * 1024, kStreamLoad);
    }
    // keep every load of the run ahead of its first use (the scheduler would
    // otherwise trade memory parallelism for registers)
    __builtin_amdgcn_sched_barrier(0);
    // every pair of the run is computed (no branch the loads could sink
    // into); a pair past the run end gets weight scale 0, which makes its
    // contribution exactly 0
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int gp = c0 + p;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        v4i bb[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w0 = h ? wv[p][c].z : wv[p][c].x, w1 = h ? wv[p][c].w : wv[p][c].y;
          bb[h] = (v4i){(int)(w0 & kNibMask), (int)((w0 << 4) & kNibMask), (int)(w1 & kNibMask),
                        (int)((w1 << 4) & kNibMask)};
        }
#pragma unroll
        for (int h = 0; h < NS; ++h) {
          const int g = NS * gp + h;                // scale group
          // sw / 16: the MFMA yields 16 * P
          const float swf = (DUMP || p >= pn) ? 0.0f : (float)t[p].sw[c][h] * 0.0625f;
          const float nsw = -kMagic * swf;
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(t[p].av[i][h], bb[h], magic, 0, 0, 0);
            if constexpr (BPG == 2)                 // the group's second block, accumulated
              d = __builtin_amdgcn_mfma_i32_16x16x64_i8(t[p].av[i][1], bb[1], d, 0, 0, 0);
            if (DUMP) {
              const int n = (nt0 + c) * 16 + colq;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int m = i * 16 + rowq + q;
                if (p < pn && g < G && m >= a.m0 && m < a.m0 + a.mc && n >= a.n0 && n < a.n0 + a.nc)
                  a.P[((size_t)(m - a.m0) * a.nc + (n - a.n0)) * G + g] = (d[q] - kMagicBits) >> 4;
              }
            } else {
              float u;
              u = __builtin_fmaf(__int_as_float(d[0]), swf, nsw);
              acc[c][i][0] = __builtin_fmaf(u, (float)t[p].sx[i][h][0], acc[c][i][0]);
              u = __builtin_fmaf(__int_as_float(d[1]), swf, nsw);
              acc[c][i][1] = __builtin_fmaf(u, (float)t[p].sx[i][h][1], acc[c][i][1]);
              u = __builtin_fmaf(__int_as_float(d[2]), swf, nsw);
              acc[c][i][2] = __builtin_fmaf(u, (float)t[p].sx[i][h][2], acc[c][i][2]);
              u = __builtin_fmaf(__int_as_float(d[3]), swf, nsw);
              acc[c][i][3] = __builtin_fmaf(u, (float)t[p].sx[i][h][3], acc[c][i][3]);
              // each MFMA result is consumed before the next MFMA issues (the
              // scheduler would otherwise keep all of them alive at once)
#pragma unroll
              for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(acc[c][i][q]));
            }
          }
        }
      }
    }
  }
  if (DUMP) return;

  // epilogue operands into LDS, loaded only now: held across the weight
  // stream they would cost registers the stream needs (the barrier below
  // orders them)
  for (int p = tid; p < EUN; p += nthr) {               // U: the slices summed in order
    const int c = p / (MT * 16), row = p % (MT * 16);
    const float *up = a.uw + ((size_t)proj * a.r + c) * a.Mpad + row;
    const size_t sstride = (size_t)a.ucols * a.Mpad;
    float us[kMaxUSlicesSkinny];                        // the first slices loaded together
#pragma unroll
    for (int sl = 0; sl < kMaxUSlicesSkinny; ++sl) us[sl] = up[(size_t)min(sl, a.u_slices - 1) * sstride];
    float u = 0.0f;
#pragma unroll
    for (int sl = 0; sl < kMaxUSlicesSkinny; ++sl)
      if (sl < a.u_slices) u += us[sl];
    for (int sl = kMaxUSlicesSkinny; sl < a.u_slices; ++sl) u += up[(size_t)sl * sstride];
    eu[p] = u;
  }
  for (int p = tid; p < ELN; p += nthr)
    el2[p] = bf16_to_f32(a.L2[((size_t)proj * a.r + p / (16 * CT)) * a.N + min(nt0 * 16 + p % (16 * CT), a.N - 1)]);
  if (tid < 16 * CT)
    eb[tid] = a.bias ? bf16_to_f32(a.bias[(size_t)proj * a.N + min(nt0 * 16 + tid, a.N - 1)]) : 0.0f;

  // ---- the W partial tiles: parked, then each output summed over the
  // waves in order, plus U * L2 and the bias ----
  constexpr int E = CT * MT * 4;                       // values per lane
  {
    float *dst = red + wave * E * 64;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[((c * MT + i) * 4 + q) * 64 + lane] = acc[c][i][q];
  }
  __syncthreads();                                      // partial tiles and epilogue operands
  for (int o = tid; o < E * 64; o += nthr) {
    const int e = o >> 6, l = o & 63;                   // value e of lane l
    const int c = e / (MT * 4), i = (e >> 2) % MT, q = e & 3;
    const int n = (nt0 + c) * 16 + (l & 15);
    const int m = i * 16 + 4 * (l >> 4) + q;
    float y = 0.0f;
    for (int w = 0; w < W; ++w) y += red[w * E * 64 + o];
    if (n >= a.N || m >= a.M) continue;
    for (int k = 0; k < a.r; ++k) y = __builtin_fmaf(eu[k * MT * 16 + m], el2[k * 16 * CT + c * 16 + (l & 15)], y);
    y += eb[c * 16 + (l & 15)];
    const size_t off = ((size_t)proj * a.M + m) * a.N + n;
    if (a.y_bf16)
      reinterpret_cast<uint16_t *>(a.Y)[off] = f32_to_bf16(y);
    else
      reinterpret_cast<float *>(a.Y)[off] = y;
  }
}

template <int MT, int P, int CT, int BPG>
hipError_t launch_cfg(const GemmArgs &a, int batch, bool dump, int W, hipStream_t s) {
  const int NT = ceil_div(a.N, kTile);
  const size_t lds = ((size_t)W * CT * MT * 4 * 64 + (size_t)a.r * MT * 16 + (size_t)a.r * 16 * CT +
                      16 * CT) * sizeof(float);
  if (dump) {
    const int g0 = a.n0 / (16 * CT), g1 = (a.n0 + a.nc - 1) / (16 * CT);
    hipLaunchKernelGGL((k_gemm_skinny<MT, P, CT, true, BPG>), dim3((unsigned)(g1 - g0 + 1), 1u),
                       dim3((unsigned)(64 * W)), 0, s, a, W);
  } else {
    hipLaunchKernelGGL((k_gemm_skinny<MT, P, CT, false, BPG>), dim3((unsigned)ceil_div(NT, CT), (unsigned)batch),
                       dim3((unsigned)(64 * W)), lds, s, a, W);
  }
  return hipGetLastError();
}

// Waves W: enough runs of P group pairs to cover K, at most max_waves(MT)
// per workgroup (longer K loops over runs, balanced).
int waves_for(int GP, int P, int mt) {
  const int runs = ceil_div(GP, P);
  return ceil_div(runs, ceil_div(runs, max_waves(mt)));
}

// One row tile: runs of 4 pairs x 1 column tile, or 2 pairs x CT column
// tiles (the activation operands of a pair then serve CT weight blocks).
// Cost = sequential runs per wave x rounds of 4096 waves (about what the
// chip holds at this register use), with a penalty when fewer workgroups
// than CUs stream; the cheapest shape wins, wider CT on ties.
template <int BPG>
hipError_t launch_mt1(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  const int NT = ceil_div(a.N, kTile), GP = a.Gp / 2;
  auto cost = [&](int P, int CT) {
    const int W = waves_for(GP, P, 1);
    const long long wgs = (long long)ceil_div(NT, CT) * batch;
    const long long waves = wgs * W;
    long long c = (long long)ceil_div(ceil_div(GP, P), W) * ((waves + 4095) / 4096) * 4;
    if (wgs < 256) c += (256 - wgs) * 4 / 256 + 1;   // idle CUs
    return c;
  };
  // (group 128 keeps both blocks of a pair unpacked at once: four column
  // tiles would not fit the register budget, so it stops at three)
  constexpr int kShapes = BPG == 1 ? 4 : 3;
  int best = 0;
  const long long cs[4] = {cost(4, 1), cost(2, 2), cost(2, 3), cost(2, 4)};
  for (int k = 1; k < kShapes; ++k)
    if (cs[k] <= cs[best]) best = k;
  switch (best) {
    case 3:
      if constexpr (BPG == 1) return launch_cfg<1, 2, 4, BPG>(a, batch, dump, waves_for(GP, 2, 1), s);
      [[fallthrough]];
    case 2: return launch_cfg<1, 2, 3, BPG>(a, batch, dump, waves_for(GP, 2, 1), s);
    case 1: return launch_cfg<1, 2, 2, BPG>(a, batch, dump, waves_for(GP, 2, 1), s);
    default: return launch_cfg<1, 4, 1, BPG>(a, batch, dump, waves_for(GP, 4, 1), s);
  }
}

template <int MT, int BPG>
hipError_t launch_mt(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  return launch_cfg<MT, 2, 1, BPG>(a, batch, dump, waves_for(a.Gp / 2, 2, MT), s);
}

template <int BPG>
hipError_t launch_bpg(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  switch (ceil_div(a.M, kTile)) {
    case 1: return launch_mt1<BPG>(a, batch, dump, s);
    case 2: return launch_mt<2, BPG>(a, batch, dump, s);
    case 3: return launch_mt<3, BPG>(a, batch, dump, s);
    case 4: return launch_mt<4, BPG>(a, batch, dump, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  return a.bpg == 2 ? launch_bpg<2>(a, batch, dump, s) : launch_bpg<1>(a, batch, dump, s);
}

}  // namespace hsq

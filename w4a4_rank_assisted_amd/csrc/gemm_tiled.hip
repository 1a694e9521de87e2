// gemm_tiled.hip -- K2 (TILED): the int4 x int4 residual contraction with an
// int32 partial sum per 64-wide group, rescaled by sx * sw in fp32, plus the
// rank-r epilogue U * L2 + bias.
//
// Operation (hsq.h formula block; W ~ L1*L2 + Q(R), Deflating the Hessian,
// abstract; group-64, Table 1 caption).
//
// One 16x16x64 int8 MFMA covers exactly one group of one 16x16 output tile.
// Operands: A = activation codes (int8, written by K1 in MFMA lane order),
// B = residual codes as int8 bytes 16*code (the packed blob's operand part,
// in MFMA lane order), so the MFMA yields 16*P.  The MFMA accumulator input
// is the bit pattern of 1.5*2^23; the result bits then read as the float
// 1.5*2^23 + 16P exactly, and two FMAs per element finish the group:
//   u   = fma(D, sw/16, -1.5*2^23*sw/16)   (= P*sw rounded once; the
//                                            constant product is exact)
//   acc = fma(u, sx, acc)                   (sx read as fp16: v_fma_mix_f32)
// Those two VALU FMAs per element and group bound the kernel: measured on
// gfx950 with all operands in registers, the 8 FMAs that follow each MFMA
// (4 elements per lane) hold the matrix core near 42 % busy (85-96 % with
// none).  So the loop spends no other VALU work per group: both operands
// move global -> LDS with direct-to-LDS buffer loads (no register staging,
// no unpacking), and within a stage the row tiles run as a software
// pipeline (LDS read one step ahead, MFMAs of step k, rescale of step k-1).
//
// Workgroup: 512 threads = 8 waves in 2 (M) x 4 (N), tile BM x BN =
// 128 x 128; each wave owns 64 x 32 outputs = 4 x 2 MFMA tiles.  A stage is
// one pair of 64-channel blocks (two groups, or one group of 128): 16 KB of
// A and 16 KB of B, four 1 KB direct-to-LDS loads per wave, in one of two
// LDS buffers.  The loads of stage s+1 are issued as stage s starts, so they
// have the whole stage to arrive; one barrier per stage (an explicit wait on
// this wave's loads and LDS writes, then s_barrier: no fence, which would
// also drain the loads in flight).  Workgroups are mapped so that each XCD
// (own L2) walks a compact block of output tiles.
//
// Split K: when the output has too few tiles to fill the chip (a few hundred
// tokens against a long K), S workgroups share a tile, each over a range of
// stages, and store their fp32 accumulators as partial tiles in the
// workspace; a second launch of the same kernel sums the S partials of a
// tile in split order (deterministic) and runs the epilogue.
//
// K halves: with a few hundred tiles or fewer, a workgroup of 16 waves may
// own a tile instead, as two 8-wave halves over the two halves of its K
// range, each with its own stage buffers; they share the stage barriers,
// and half 1 hands its accumulators to half 0 through LDS at the end (a
// fixed order, no workspace traffic).  tiled_plan picks halves and splits
// from a cost model fitted to measured times.
#include "hsq_internal.h"

#include <cstddef>
#include <type_traits>

namespace hsq {

namespace {

constexpr int BM = 128, BN = 128;
constexpr int TMB = BM / 16, TNB = BN / 16;   // MFMA tiles per block
constexpr int WM = 2, WN = 4;                 // waves along M and N
constexpr int NTH = 64 * WM * WN;             // threads per workgroup
constexpr int TM = TMB / WM, TN = TNB / WN;   // MFMA tiles per wave (64 x 32 outputs)
constexpr int kGroupM = 8;                    // m-blocks per tile-order group
// kernel modes: the whole K range with the epilogue, one split's partial
// tile, or the sum of the partial tiles with the epilogue
constexpr int kFull = 0, kSplit = 1, kReduce = 2;
constexpr int kCUs = 256;                     // compute units of the MI355X
constexpr int kMaxSplits = 16;
constexpr int kMinSplitStages = 4;            // stages (block pairs) per split, at least
constexpr int kAccPerThread = TM * TN * 4;
static_assert(TMB == WM * WN && TNB == WM * WN, "one A and one B tile per wave and block");
static_assert(TMB * 16 == 128 && BN == 128, "scale staging: 128 values per scale group and two waves");

// One stage is one pair of 64-channel blocks: two scale groups (BPG = 1,
// group 64) or one (BPG = 2, group 128).
template <int BPG>
struct alignas(16) Stages {
  static constexpr int SPS = 2 / BPG;  // scale groups per stage
  int8_t a[2][2][TMB][64][16];         // [buf][block][m-tile][lane][bytes]   16 KB per buffer
  int8_t b[2][2][TNB][64][16];         // [buf][block][n-tile][lane][bytes]   16 KB per buffer
  float2 sw[2][2][BN];                 // [buf][group][col] = (sw, -magic*sw)/16          2 KB per buffer
  uint16_t sx[2][TMB][2][16];          // [buf][m-tile][group][row] fp16                 512 B per buffer
};
static_assert(offsetof(Stages<1>, a) == 0 && offsetof(Stages<1>, b) == sizeof(Stages<1>::a) &&
              offsetof(Stages<2>, a) == 0 && offsetof(Stages<2>, b) == sizeof(Stages<2>::a),
              "the direct-to-LDS addresses assume A then B at the start of a stage set");
static_assert(sizeof(Stages<1>::sw[0][0]) == 1024 && sizeof(Stages<1>::sx[0]) == 512,
              "one direct-to-LDS load per scale group of weight scales, half of one for the activation scales");

// Epilogue operands of the block: U (rank columns padded to RPT) for its
// BM rows, L2 for its BN columns, bias.  Filled at kernel start.
template <int RPT>
struct alignas(16) EpiSmem {
  float u[RPT][BM];
  float l2[RPT][BN];
  float bias[BN];
};
template <>
struct alignas(16) EpiSmem<0> {
  float bias[BN];
};

// KH = 2: two halves of 8 waves share the tile, each with its own stage
// buffers and half of the K range; half 1 parks its accumulators at
// kRedOff (past the output-transpose area of half 0's waves) once the
// stage loop is over.
constexpr int kRedOff = WM * WN * 16 * (TN * 16) * 4;   // bytes
template <int RPT, int BPG, int KH>
struct alignas(16) Smem {
  union {
    Stages<BPG> st[KH];
    float red[KH == 2 ? kRedOff / 4 + NTH * TM * TN * 4 : 1];
  };
  EpiSmem<RPT> ep;
};

template <int V>
struct int_c {
  static constexpr int value = V;
};

// Order pins.  An empty volatile asm that "rewrites" a register value makes
// every later use depend on it, and volatile asm statements keep their
// program order; the pins below fix the software pipeline that the
// instruction selector would otherwise flatten into all-MFMAs-first, which
// keeps every MFMA result alive at once and spills.
__device__ __forceinline__ void pin(v4i &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

template <bool DUMP, int RPT, int MODE, int BPG, int KH, bool CHAIN = false>
__global__ __launch_bounds__(NTH * KH, 4) void k_gemm_tiled(GemmArgs a, int nblk, int mblk) {
  static_assert(MODE != kSplit || RPT == 0, "a split pass has no epilogue");
  static_assert(KH == 1 || (!DUMP && MODE != kReduce), "the K halves serve the stage loop");
  static_assert(!CHAIN || (MODE == kFull && KH == 1 && BPG == 1 && !DUMP), "the chain epilogue: one unsplit pass");
  constexpr bool EPI = !DUMP && MODE != kSplit;   // this pass writes Y
  constexpr int SPS = Stages<BPG>::SPS;           // scale groups per stage
  constexpr int NSTEP = SPS * TM;                 // pipeline steps per stage (one row tile and scale group each)
  __shared__ Smem<RPT, BPG, KH> smem;

  const int lane = threadIdx.x & 63;
  const int wave0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int half = KH == 1 ? 0 : wave0 / (WM * WN);   // K half of this wave
  const int tid = (int)threadIdx.x - half * NTH;     // thread index within the half
  const int wave = wave0 - half * (WM * WN);
  Stages<BPG> &sm = smem.st[half];
  const int wm = wave / WN, wn = wave % WN;
  const int proj = blockIdx.y;
  int mb, nb;
  xcd_tile_of(blockIdx.x, nblk, mblk, kGroupM, mb, nb);
  const int mt0 = mb * TMB, nt0 = nb * TNB;
  const int MT = a.Mpad / 16, NT = (a.N + 15) / 16;
  const uint8_t *w = a.w + (size_t)proj * a.w_stride + a.w_ops;   // int8 operand part
  const uint16_t *sw = DUMP ? nullptr : a.sw + (size_t)proj * a.G * a.N;
  if (DUMP && ((mt0 + TMB) * 16 <= a.m0 || mt0 * 16 >= a.m0 + a.mc ||
               (nt0 + TNB) * 16 <= a.n0 || nt0 * 16 >= a.n0 + a.nc))
    return;  // whole block outside the window (uniform: before any barrier)
  // stages: block pairs, [s0, s1): all of them, or one split's range
  const int nst = a.Gp / 2;
  int s0 = 0, s1 = nst;
  if (MODE == kSplit) {
    const int S = (int)gridDim.z, z = (int)blockIdx.z;
    s0 = z * nst / S;
    s1 = (z + 1) * nst / S;
  }
  // stages with data for this workgroup end at send; with two K halves,
  // half h runs [s0 + h*L, s0 + (h+1)*L), so both make the same number of
  // steps (barriers); stages of half 1 past send get weight scale 0 and
  // add exactly 0
  const int send = s1;
  if constexpr (KH == 2) {
    const int L = (s1 - s0 + 1) / 2;
    s0 += half * L;
    s1 = s0 + L;
  }
  // this tile's partial tiles: [proj][tile][split][chunk][thread] float4
  float *part_tile = a.part + (((size_t)proj * nblk * mblk + (size_t)mb * nblk + nb) * a.splits) *
                                  (NTH * kAccPerThread);

  // ---- global -> LDS ----
  // Operand blocks: wave w moves A block (row tile mt0 + w) and B block
  // (column tile nt0 + w) for both blocks of the stage's pair.  Tiles past
  // the matrix edges load the last real tile (clamped: straight-line code);
  // their rows and columns are masked by zero scales and at the store.
  const int G = a.G;                  // scale groups
  const v4u rs_a = raw_rsrc(a.qa, (uint32_t)MT * a.Gp * 1024);
  const v4u rs_w = raw_rsrc(w, (uint32_t)NT * a.Gp * 1024);
  const v4u rs_x = raw_rsrc(a.sxs, (uint32_t)MT * a.SG * 32);
  const uint32_t swp_bytes = (uint32_t)a.swr * (uint32_t)a.npad * 8u;
  const v4u rs_p = raw_rsrc(DUMP ? nullptr : (const char *)a.swp + (size_t)proj * swp_bytes, DUMP ? 0u : swp_bytes);
  const uint32_t offa = ((uint32_t)min(mt0 + wave, MT - 1) * a.Gp * 64 + lane) * 16;
  const uint32_t offb = ((uint32_t)min(nt0 + wave, NT - 1) * a.Gp * 64 + lane) * 16;
  // scales: wave 0's first 32 lanes move the activation scales of the
  // stage's two 64-channel groups for the 8 row tiles (64 bytes per tile,
  // 16 per lane), waves 1 .. SPS the weight-scale pairs of one scale group
  // for the 128 columns (1 KB); stages past the workgroup's range read the
  // zero rows of the pair array, so they add exactly 0
  const uint32_t offsx = (uint32_t)min(mt0 + (lane >> 2), MT - 1) * a.SG * 32 + (uint32_t)(lane & 3) * 16;
  const uint32_t offsw = (uint32_t)nt0 * 16 * 8 + (uint32_t)lane * 16;
  const int swg = BPG == 1 ? a.Gp : G;     // scale groups of the pair array before its zero rows
  const int last = nst - 1;
  // LDS byte addresses of this wave's A and B blocks in buffer 0, block 0
  // (the stage buffers open the shared object; a buffer is 2 x 8 KB per
  // operand), and of the scales
  const uint32_t lds_st = lds_addr(&smem) + (uint32_t)half * (uint32_t)sizeof(Stages<BPG>);
  const uint32_t lds_a = lds_st + (uint32_t)wave * 1024;
  const uint32_t lds_b = lds_st + (uint32_t)offsetof(Stages<BPG>, b) + (uint32_t)wave * 1024;
  const uint32_t lds_sw = lds_st + (uint32_t)offsetof(Stages<BPG>, sw);
  const uint32_t lds_sx = lds_st + (uint32_t)offsetof(Stages<BPG>, sx);
  auto load_stage = [&](int st, int buf) __attribute__((always_inline)) {
    const int sl = min(st, last);     // past the end: a clamped reload (its weight scales are 0)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint32_t blk = (uint32_t)(buf * 2 + b) * TMB * 1024;
      block_to_lds(rs_a, lds_a + blk, offa, (uint32_t)(2 * sl + b) * 1024);
      block_to_lds(rs_w, lds_b + blk, offb, (uint32_t)(2 * sl + b) * 1024);
    }
    if (wave == 0) {
      if (lane < 32) block_to_lds(rs_x, lds_sx + (uint32_t)buf * 512, offsx, (uint32_t)(SPS * sl) * 32);
    } else if (!DUMP && wave <= SPS) {
      const int sg = wave - 1;
      const int row = st < send ? SPS * st + sg : swg + sg;
      block_to_lds(rs_p, lds_sw + (uint32_t)(buf * 2 + sg) * 1024, offsw, (uint32_t)row * (uint32_t)a.npad * 8u);
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

  // ---- epilogue operands: loads issued first, so that their latency
  // overlaps the first stage's loads; parked in LDS below ----
  constexpr int EU = RPT * BM / NTH;  // (rank column, row) pairs per thread
  constexpr int US = RPT <= 8 ? kMaxUSlices : kMaxUSlices / 2;  // U slices prefetched
  float eu[EU > 0 ? EU : 1][US], el2[EU > 0 ? EU : 1], ebias = 0.0f;
  if (EPI && half == 0) {
    const uint16_t *L2 = a.L2 + (size_t)proj * a.r * a.N;
#pragma unroll
    for (int e = 0; e < EU; ++e) {
      const int idx = e * NTH + tid, c = idx / BM, rr = idx % BM;
      const int cc = min(c, a.r - 1);
      const int m = min(mt0 * 16 + rr, a.Mpad - 1);
#pragma unroll
      for (int sl = 0; sl < US; ++sl)
        eu[e][sl] = a.uw[((size_t)min(sl, a.u_slices - 1) * a.ucols + (size_t)proj * a.r + cc) * a.Mpad + m];
      el2[e] = bf16_to_f32(L2[(size_t)cc * a.N + min(nt0 * 16 + rr, a.N - 1)]);
    }
    if (a.bias) ebias = bf16_to_f32(a.bias[(size_t)proj * a.N + min(nt0 * 16 + (tid & (BN - 1)), a.N - 1)]);
  }

  if constexpr (MODE != kReduce) load_stage(s0, 0);
  if (EPI && half == 0) {
#pragma unroll
    for (int e = 0; e < EU; ++e) {
      const int idx = e * NTH + tid, c = idx / BM, rr = idx % BM;
      float u = 0.0f;
#pragma unroll
      for (int sl = 0; sl < US; ++sl) u += sl < a.u_slices ? eu[e][sl] : 0.0f;
      if (a.u_slices > US) {              // long K: the remaining slices, in order
        const int cc = min(c, a.r - 1), m = min(mt0 * 16 + rr, a.Mpad - 1);
        for (int sl = US; sl < a.u_slices; ++sl)
          u += a.uw[((size_t)sl * a.ucols + (size_t)proj * a.r + cc) * a.Mpad + m];
      }
      const bool live = c < a.r;
      if constexpr (RPT > 0) {
        smem.ep.u[c][rr] = (live && mt0 * 16 + rr < a.M) ? u : 0.0f;
        smem.ep.l2[c][rr] = (live && nt0 * 16 + rr < a.N) ? el2[e] : 0.0f;
      }
    }
    if (tid < BN) smem.ep.bias[tid] = (nt0 * 16 + tid < a.N) ? ebias : 0.0f;
  }
  stage_barrier();

  if constexpr (MODE != kReduce) {

  // ---- the stage loop, software-pipelined across steps and stages.  Step
  // k of a stage (row tile k % TM of scale group k / TM) issues its MFMAs
  // and rescales step k-1: a step of this stage, or, at k = 0, the last
  // step of the previous stage (its MFMA results, weight scales and
  // activation scales are carried over; its FMAs go first, while the
  // stage's first LDS reads are in flight), so the pipeline never drains
  // at a stage boundary.
  v4i d[TM][TN];                      // MFMA results (row TM-1 carried)
  float2 swc[TN];                     // weight scales of the carried step
  v4h sxc;                            // activation scales of the carried step
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    d[TM - 1][j] = magic;             // a first carry that adds exactly 0
    swc[j] = make_float2(0.0f, 0.0f);
  }
  sxc = (v4h){0, 0, 0, 0};

  // rescale one row tile: acc += (D - magic) * sw * sx, or, for the test
  // export, the group partials of the window
  auto rescale = [&](int ip, const float2 (&sw2)[TN], const v4h sx4, int gg)
      __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if (DUMP) {
        const int n = (nt0 + wn * TN + j) * 16 + colq;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = (mt0 + wm * TM + ip) * 16 + rowq + q;
          if (gg >= 0 && gg < G && m >= a.m0 && m < a.m0 + a.mc && n >= a.n0 && n < a.n0 + a.nc)
            a.P[((size_t)(m - a.m0) * a.nc + (n - a.n0)) * G + gg] = (d[ip][j][q] - kMagicBits) >> 4;
        }
      } else {
        const float2 s2 = sw2[j];
        const float u0 = __builtin_fmaf(__int_as_float(d[ip][j][0]), s2.x, s2.y);
        const float u1 = __builtin_fmaf(__int_as_float(d[ip][j][1]), s2.x, s2.y);
        const float u2 = __builtin_fmaf(__int_as_float(d[ip][j][2]), s2.x, s2.y);
        const float u3 = __builtin_fmaf(__int_as_float(d[ip][j][3]), s2.x, s2.y);
        acc[ip][j][0] = __builtin_fmaf(u0, (float)sx4.x, acc[ip][j][0]);
        acc[ip][j][1] = __builtin_fmaf(u1, (float)sx4.y, acc[ip][j][1]);
        acc[ip][j][2] = __builtin_fmaf(u2, (float)sx4.z, acc[ip][j][2]);
        acc[ip][j][3] = __builtin_fmaf(u3, (float)sx4.w, acc[ip][j][3]);
      }
    }
    if (!DUMP) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) pin(acc[ip][j][q]);
    }
  };

  auto stage = [&](int st, auto bufc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;    // LDS buffer == (st - s0) & 1
    // the next stage's operands and scales: in flight during this stage
    // (past the end: a clamped, unused reload)
    load_stage(st + 1, BUF ^ 1);

    v4i bv[2][TN];                    // B operands of the pair's blocks
    float2 swv[SPS][TN];              // weight scales of the stage's scale groups
    v4i av[NSTEP][BPG];
    v4h sxv[NSTEP];
    auto read_b = [&](int b) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bv[b][j] = *reinterpret_cast<const v4i *>(&sm.b[BUF][b][wn * TN + j][lane][0]);
    };
    auto read_step = [&](int k) __attribute__((always_inline)) {
      const int sg = k / TM, s = k % TM;
#pragma unroll
      for (int bb = 0; bb < BPG; ++bb)
        av[k][bb] = *reinterpret_cast<const v4i *>(&sm.a[BUF][sg * BPG + bb][wm * TM + s][lane][0]);
      sxv[k] = *reinterpret_cast<const v4h *>(&sm.sx[BUF][wm * TM + s][sg][rowq]);
    };
    // one step's MFMAs: a group-128 scale group's two blocks accumulate in
    // int32 (the second MFMA takes the first one's result as its input)
    auto mfma_step = [&](int k) __attribute__((always_inline)) {
      const int sg = k / TM, s = k % TM;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        d[s][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[k][0], bv[sg * BPG][j], magic, 0, 0, 0);
        if constexpr (BPG == 2)
          d[s][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[k][1], bv[1][j], d[s][j], 0, 0, 0);
      }
    };
    read_b(0);
#pragma unroll
    for (int sg = 0; sg < SPS; ++sg)
#pragma unroll
      for (int j = 0; j < TN; ++j) swv[sg][j] = sm.sw[BUF][sg][(wn * TN + j) * 16 + colq];
    read_step(0);
    if constexpr (BPG == 2) read_b(1);
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      // step boundary: nothing moves across it
      __builtin_amdgcn_sched_barrier(0);
      if (k == 0) {
        // the carried step first: its FMAs need no LDS data, so they cover
        // the latency of this stage's first reads (issued just above)
        if (NSTEP > 1) read_step(1);
        rescale(TM - 1, swc, sxc, st * SPS - 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bb = 0; bb < BPG; ++bb) pin(av[0][bb]);
        mfma_step(0);
        continue;
      }
#pragma unroll
      for (int bb = 0; bb < BPG; ++bb) pin(av[k][bb]);
      if (k + 1 < NSTEP) read_step(k + 1);
      if (BPG == 1 && k == TM - 1) read_b(1);     // the second block's B, one step ahead
      mfma_step(k);
      rescale((k - 1) % TM, swv[(k - 1) / TM], sxv[k - 1], st * SPS + (k - 1) / TM);
      // issue order within the step: one tile's MFMAs, then the eight
      // rescale FMAs of one tile, and so on, so the matrix core works while
      // the VALU rescales
      if (!DUMP) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, BPG, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < TN; ++j) swc[j] = swv[SPS - 1][j];
    sxc = sxv[NSTEP - 1];

    stage_barrier();
  };
  // stages in pairs (compile-time LDS buffers), then an odd last one
  int st = s0;
  for (; st + 2 <= s1; st += 2) {
    stage(st, int_c<0>{});
    stage(st + 1, int_c<1>{});
  }
  if (st < s1) stage(st, int_c<0>{});
  // drain: the last step of the last stage
  rescale(TM - 1, swc, sxc, s1 * SPS - 1);
  }  // MODE != kReduce

  if (DUMP) return;

  if constexpr (KH == 2) {
    // half 1's accumulators to LDS (the stage loop ended with a barrier, so
    // the stage buffers are free), added by half 0 in a fixed order
    float *red = smem.red + kRedOff / 4;
    if (half == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          *reinterpret_cast<v4f *>(red + ((i * TN + j) * NTH + tid) * 4) =
              (v4f){acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
    }
    __syncthreads();
    if (half == 1) return;            // no barrier follows
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f v = *reinterpret_cast<const v4f *>(red + ((i * TN + j) * NTH + tid) * 4);
        acc[i][j][0] += v[0]; acc[i][j][1] += v[1]; acc[i][j][2] += v[2]; acc[i][j][3] += v[3];
      }
  }

  if constexpr (MODE == kSplit) {
    // this split's partial tile: chunk c = (i, j) as one float4 per thread,
    // 1 KB contiguous per wave and chunk
    float *dst = part_tile + (size_t)blockIdx.z * (NTH * kAccPerThread);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        *reinterpret_cast<v4f *>(dst + ((i * TN + j) * NTH + tid) * 4) =
            (v4f){acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
    return;
  }
  if constexpr (MODE == kReduce) {
    // the partial tiles in split order
#pragma unroll 1
    for (int z = 0; z < a.splits; ++z) {
      const float *src = part_tile + (size_t)z * (NTH * kAccPerThread);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v4f v = *reinterpret_cast<const v4f *>(src + ((i * TN + j) * NTH + tid) * 4);
          acc[i][j][0] += v[0]; acc[i][j][1] += v[1]; acc[i][j][2] += v[2]; acc[i][j][3] += v[3];
        }
    }
  }

  // ---- epilogue: Y = acc + U * L2 + bias ----
  // U * L2 as fp32 MFMAs (16x16x4: one per 16x16 tile and 4 rank columns);
  // the stage loop ended with a barrier (the reduce pass has none: its
  // stage buffers were never used), so that LDS is free for the output
  // transpose.
  if constexpr (RPT > 0) {
#pragma unroll
  for (int cc = 0; cc < RPT / 4; ++cc) {
    float ua[TM], lb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) ua[i] = smem.ep.u[cc * 4 + (lane >> 4)][(wm * TM + i) * 16 + colq];
#pragma unroll
    for (int j = 0; j < TN; ++j) lb[j] = smem.ep.l2[cc * 4 + (lane >> 4)][(wn * TN + j) * 16 + colq];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        v4f c4 = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        c4 = __builtin_amdgcn_mfma_f32_16x16x4f32(ua[i], lb[j], c4, 0, 0, 0);
        acc[i][j][0] = c4[0]; acc[i][j][1] = c4[1]; acc[i][j][2] = c4[2]; acc[i][j][3] = c4[3];
      }
  }
  }
  float bj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) bj[j] = smem.ep.bias[(wn * TN + j) * 16 + colq];

  if constexpr (CHAIN) {
    // ---- fused chain: the next layer's input instead of Y ----
    // x = act(Y) * fl32(1 / lam2[n]) (0 past M or N); per row and 64-column
    // group (the columns of a pair of waves) the scale and codes exactly as
    // the quantization pass forms them, the codes written to the next
    // layer's workspace in MFMA operand order; the partial sums of the next
    // layer's rank-r2 down projection over this tile's 128 columns.  The
    // stage buffers are free (the stage loop ended with a barrier):
    //   [0, 16 KiB)        codes, [wave][row][column] int8
    //   [16, 18 KiB)       row absmax, [wave][row]
    //   [18, 34 KiB)       U shares, [column quarter][tile row][8]
    constexpr int WR = TM * 16, WC = TN * 16;          // 64 rows x 32 columns per wave
    constexpr int R2 = kChainMaxRank;
    static_assert(WC == 32 && WN == 4 && BN == 128, "a 64-column group is the columns of two waves");
    static_assert(8 * WR * WC + 8 * WR * 4 + WN * BM * R2 * 4 <= (int)sizeof(Stages<BPG>), "chain LDS");
    char *lb = reinterpret_cast<char *>(&sm);
    int8_t *cbuf = reinterpret_cast<int8_t *>(lb) + wave * (WR * WC);
    float *amx = reinterpret_cast<float *>(lb + 8 * WR * WC);
    float *uex = amx + 8 * WR;
    float il[TN], l1n[TN][R2];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = (nt0 + wn * TN + j) * 16 + colq;
      il[j] = n < a.N ? 1.0f / f16_to_f32(a.lam2[n]) : 0.0f;
#pragma unroll
      for (int c = 0; c < R2; ++c)
        l1n[j][c] = (n < a.N && c < a.r2) ? bf16_to_f32(a.L1n[(size_t)n * a.r2 + c]) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tr = (wm * TM + i) * 16 + rowq + q;   // row within the tile
        const int m = mt0 * 16 + tr;
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float y = acc[i][j][q] + bj[j];
          const int n = (nt0 + wn * TN + j) * 16 + colq;
          if (a.yhid && m < a.M && n < a.N) a.yhid[(size_t)m * a.N + n] = y;
          const float v = a.act == kActGeluTanh ? gelu_tanh_f32(y) : y;
          const float x = m < a.M ? v * il[j] : 0.0f;
          acc[i][j][q] = x;
          mx = fmaxf(mx, fabsf(x));
        }
        mx = row16_max(mx);                             // over the 16 lanes holding this row's columns
        if (colq == 0) amx[wave * WR + i * 16 + rowq + q] = mx;
#pragma unroll
        for (int c = 0; c < R2; ++c) {
          if (c >= a.r2) break;
          float p = acc[i][0][q] * l1n[0][c];
#pragma unroll
          for (int j = 1; j < TN; ++j) p = __builtin_fmaf(acc[i][j][q], l1n[j][c], p);
          p = row16_sum(p);
          if (colq == 0) uex[(wn * BM + tr) * R2 + c] = p;
        }
      }
    __syncthreads();
    const int grp = 2 * nb + (wn >> 1);                 // 64-column group of the next layer
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int wr = i * 16 + rowq + q;
        const float gmax = fmaxf(amx[wave * WR + wr], amx[(wave ^ 1) * WR + wr]);
        const uint16_t s16 = act_scale16(gmax);
        const float inv_s = s16 != 0 ? 1.0f / f16_to_f32(s16) : 0.0f;
#pragma unroll
        for (int j = 0; j < TN; ++j)
          cbuf[wr * WC + j * 16 + colq] = (int8_t)(act_code_bits(acc[i][j][q], inv_s) & 0xFF);
        const int m = mt0 * 16 + wm * WR + wr;
        if ((wn & 1) == 0 && colq == 0 && m < a.Mpad && grp < a.Gp2)
          a.sxs2[((size_t)(m >> 4) * a.Gp2 + grp) * 16 + (m & 15)] = s16;
      }
    // codes: per row of the wave, two 16-channel chunks (channels
    // 32 * (wn & 1) + 16 * ch .. + 15 of the group) -> lane slot
    // (row % 16) + 16 * kq of the block (row tile, group)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = lane + 64 * k, wr = t & 63, ch = t >> 6;
      const int m = mt0 * 16 + wm * WR + wr;
      const v4u v = *reinterpret_cast<const v4u *>(cbuf + wr * WC + 16 * ch);
      if (m < a.Mpad && grp < a.Gp2) {
        const int kq = 2 * (wn & 1) + ch;
        *reinterpret_cast<v4u *>(a.qa2 + (((size_t)(m >> 4) * a.Gp2 + grp) * 64 + (m & 15) + 16 * kq) * 16) = v;
      }
    }
    // U shares of the tile: the four column quarters summed in order
    if (wn == 0) {
      for (int t = lane; t < WR * R2; t += 64) {
        const int wr = t / R2, c = t % R2;
        const int tr = wm * WR + wr, m = mt0 * 16 + tr;
        if (c < a.r2 && m < a.Mpad) {
          float u = uex[tr * R2 + c];
#pragma unroll
          for (int w = 1; w < WN; ++w) u += uex[(w * BM + tr) * R2 + c];
          a.upart2[((size_t)nb * a.r2 + c) * a.Mpad + m] = u;
        }
      }
    }
    return;
  }

  // output: per row tile, transpose the wave's 16 x 64 values through a
  // wave-private LDS region and store 16 bytes per lane
  constexpr int WC = TN * 16;                         // columns of the wave
  char *tbuf = reinterpret_cast<char *>(&sm) + wave * (16 * WC * 4);
  const int ybytes = a.y_bf16 ? 2 : 4;
  const int per16 = 16 / ybytes;                      // values per 16-byte chunk
  const bool vec_ok = (a.N % per16) == 0;
  const int ncol0 = (nt0 + wn * TN) * 16;             // first column of the wave
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int mrow0 = (mt0 + wm * TM + i) * 16;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float y = acc[i][j][q] + bj[j];
        const int off = (rowq + q) * WC + j * 16 + colq;  // [row][col] in the 16 x WC tile
        if (a.y_bf16)
          reinterpret_cast<uint16_t *>(tbuf)[off] = f32_to_bf16(y);
        else
          reinterpret_cast<float *>(tbuf)[off] = y;
      }
    // 16 rows x WC columns; chunk k of the tile = (row k / cpr, chunk k % cpr)
    const int cpr = WC / per16;                         // chunks per row
    for (int k = lane; k < 16 * cpr; k += 64) {
      const int row = k / cpr, ch = k % cpr;
      const int m = mrow0 + row, n = ncol0 + ch * per16;
      if (m >= a.M) continue;
      const v4u v = *reinterpret_cast<const v4u *>(tbuf + (row * WC + ch * per16) * ybytes);
      char *dst = reinterpret_cast<char *>(a.Y) + (((size_t)proj * a.M + m) * a.N + n) * ybytes;
      if (vec_ok && n + per16 <= a.N) {
        *reinterpret_cast<v4u *>(dst) = v;
      } else if (a.y_bf16) {  // ragged N: element stores
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < a.N)
            reinterpret_cast<uint16_t *>(dst)[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) reinterpret_cast<uint32_t *>(dst)[e] = v[e];
      }
    }
  }
}

template <int RPT, int MODE, int BPG, int KH>
hipError_t launch_rpt(const GemmArgs &a, int batch, int nblk, int mblk, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_tiled<false, RPT, MODE, BPG, KH>), dim3((unsigned)(nblk * mblk), (unsigned)batch),
                     dim3(NTH * KH), 0, s, a, nblk, mblk);
  return hipGetLastError();
}

template <int MODE, int BPG, int KH>
hipError_t launch_epi(const GemmArgs &a, int batch, int nblk, int mblk, hipStream_t s) {
  if (a.r == 0) return launch_rpt<0, MODE, BPG, KH>(a, batch, nblk, mblk, s);
  if (a.r <= 4) return launch_rpt<4, MODE, BPG, KH>(a, batch, nblk, mblk, s);
  if (a.r <= 8) return launch_rpt<8, MODE, BPG, KH>(a, batch, nblk, mblk, s);
  if (a.r <= 16) return launch_rpt<16, MODE, BPG, KH>(a, batch, nblk, mblk, s);
  // two K halves with a rank above 16 exceed the LDS (tiled_plan never asks)
  if constexpr (KH == 2) return hipErrorInvalidValue;
  else return launch_rpt<32, MODE, BPG, KH>(a, batch, nblk, mblk, s);
}

struct TiledPlan {
  int splits;   // workgroups per output tile (partial tiles in the workspace when > 1)
  int kh;       // K halves inside a workgroup (1: 8 waves, 2: 16 waves)
};

// Plan of the tiled contraction: the (K halves, splits) pair with the
// least modelled time.  Units: the time a CU running two eight-wave
// workgroups takes for one tile and one stage (a 128-channel block pair);
// each of the two then advances at half that rate.  The other constants
// are fitted to measured contraction times: one eight-wave workgroup alone
// on a CU needs 1.4 units per stage plus 1.2 for its prologue and epilogue
// (nothing else hides them); a sixteen-wave workgroup (two K halves, one
// per CU) needs 1.2 per stage, its stages rounded up to even so the halves
// match, plus 2.3 (its halves share every barrier, and half 0 alone runs
// the epilogue).  It therefore pays only where the alternative is a split:
// each split tile beyond the first writes and reads a 64 KB fp32 partial
// tile, about 0.03 units at the HBM rate such traffic reaches.  Sixteen
// waves need two sets of stage buffers (2 x 69 KB of LDS): with the
// epilogue operands of a rank above 16 they do not fit the CU's 160 KB, and
// group 128 keeps eight waves.
TiledPlan tiled_plan(int M, int N, int K, int r, int batch, int group) {
  const long long tiles = (long long)ceil_div(N, BN) * ceil_div(M, BM) * batch;
  const int stages = padded_groups(K) / 2;
  const int max_kh = (group == kGroup && r <= 16) ? 2 : 1;
  TiledPlan best{1, 1};
  double best_t = -1.0;
  for (int kh = 1; kh <= max_kh; ++kh)
    for (int S = 1; S <= kMaxSplits && (S == 1 || S * kMinSplitStages <= stages); ++S) {
      const long long wgs = tiles * S;
      const double per = (double)ceil_div(stages, S);
      double t;
      if (kh == 1)
        t = wgs <= kCUs ? 1.4 * per + 1.2 : 2.0 * (double)((wgs + 2 * kCUs - 1) / (2 * kCUs)) * per;
      else
        t = (double)((wgs + kCUs - 1) / kCUs) * (1.2 * (double)(2 * ceil_div((int)per, 2)) + 2.3);
      if (S > 1) t += 0.03 * (double)wgs;
      if (best_t < 0.0 || t < best_t - 1e-9) {
        best = {S, kh};
        best_t = t;
      }
    }
  return best;
}

}  // namespace

int tiled_splits(int M, int N, int K, int r, int batch, int group) {
  return tiled_plan(M, N, K, r, batch, group).splits;
}

size_t tiled_partial_bytes(int M, int N, int K, int r, int batch, int group) {
  const int S = tiled_splits(M, N, K, r, batch, group);
  if (S <= 1) return 0;
  return (size_t)S * ceil_div(N, BN) * ceil_div(M, BM) * batch * NTH * kAccPerThread * sizeof(float);
}

template <int BPG, int KH>
hipError_t launch_tiled_kh(const GemmArgs &a, int batch, int S, int nblk, int mblk, hipStream_t s) {
  if (S <= 1) return launch_epi<kFull, BPG, KH>(a, batch, nblk, mblk, s);
  GemmArgs b = a;
  b.splits = S;
  hipLaunchKernelGGL((k_gemm_tiled<false, 0, kSplit, BPG, KH>),
                     dim3((unsigned)(nblk * mblk), (unsigned)batch, (unsigned)S), dim3(NTH * KH), 0, s, b,
                     nblk, mblk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_epi<kReduce, BPG, 1>(b, batch, nblk, mblk, s);
}

template <int BPG>
hipError_t launch_tiled_bpg(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  const int nblk = ceil_div(a.N, BN), mblk = ceil_div(a.M, BM);
  if (dump) {
    // every tile of one projection; blocks outside the window exit at once
    hipLaunchKernelGGL((k_gemm_tiled<true, 0, kFull, BPG, 1>), dim3((unsigned)(nblk * mblk), 1u), dim3(NTH),
                       0, s, a, nblk, mblk);
    return hipGetLastError();
  }
  const TiledPlan p = tiled_plan(a.M, a.N, a.G * kGroup * BPG, a.r, batch, kGroup * BPG);
  if constexpr (BPG == 1)
    if (p.kh == 2) return launch_tiled_kh<BPG, 2>(a, batch, p.splits, nblk, mblk, s);
  return launch_tiled_kh<BPG, 1>(a, batch, p.splits, nblk, mblk, s);
}

// The weight-scale pairs of the stage loop (sw_pair_item), one thread per 8
// pairs; the linear writes them from its quantization pass instead.
__global__ __launch_bounds__(256) void k_sw_pairs(const uint16_t *__restrict__ sw, int G, int N, int swr, int npad,
                                                  size_t total8, float4 *__restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < total8) sw_pair_item(sw, G, N, swr, npad, i, out);
}

template <int RPT>
hipError_t launch_chain_rpt(const GemmArgs &a, int nblk, int mblk, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_tiled<false, RPT, kFull, 1, 1, true>), dim3((unsigned)(nblk * mblk), 1u), dim3(NTH),
                     0, s, a, nblk, mblk);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_chain_ureduce(const float *upart, int nblk, int r2, int Mpad, float *uw) {
  const int i = blockIdx.x * 256 + threadIdx.x;     // (rank column, row) of the next layer's U
  if (i >= r2 * Mpad) return;
  float u = 0.0f;
#pragma unroll 8
  for (int b = 0; b < nblk; ++b) u += upart[(size_t)b * r2 * Mpad + i];
  uw[i] = u;
}

hipError_t launch_gemm_tiled_chain(const GemmArgs &a, hipStream_t s) {
  if (a.bpg != 1 || a.r2 < 0 || a.r2 > kChainMaxRank) return hipErrorInvalidValue;
  const int nblk = ceil_div(a.N, BN), mblk = ceil_div(a.M, BM);
  if (a.r == 0) return launch_chain_rpt<0>(a, nblk, mblk, s);
  if (a.r <= 4) return launch_chain_rpt<4>(a, nblk, mblk, s);
  if (a.r <= 8) return launch_chain_rpt<8>(a, nblk, mblk, s);
  if (a.r <= 16) return launch_chain_rpt<16>(a, nblk, mblk, s);
  return launch_chain_rpt<32>(a, nblk, mblk, s);
}

hipError_t launch_chain_ureduce(const float *upart, int nblk, int r2, int Mpad, float *uw, hipStream_t s) {
  hipLaunchKernelGGL(k_chain_ureduce, dim3((unsigned)ceil_div(r2 * Mpad, 256)), dim3(256), 0, s, upart, nblk, r2,
                     Mpad, uw);
  return hipGetLastError();
}

hipError_t launch_sw_pairs(const GemmArgs &a, int batch, hipStream_t s) {
  const size_t total8 = (size_t)batch * a.swr * (a.npad / 8);
  hipLaunchKernelGGL(k_sw_pairs, dim3((unsigned)((total8 + 255) / 256)), dim3(256), 0, s, a.sw, a.G, a.N, a.swr,
                     a.npad, total8, reinterpret_cast<float4 *>(const_cast<float2 *>(a.swp)));
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const GemmArgs &a, int batch, bool dump, hipStream_t s) {
  return a.bpg == 2 ? launch_tiled_bpg<2>(a, batch, dump, s) : launch_tiled_bpg<1>(a, batch, dump, s);
}

}  // namespace hsq

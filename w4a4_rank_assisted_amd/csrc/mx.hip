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

namespace hsq {

namespace {

constexpr int MB = 128, NB = 128;                 // output tile
constexpr int MTB = MB / 16, NTB = NB / 16;      // MFMA tiles per output tile
constexpr int MWM = 2, MWN = 4;                   // waves along M and N
constexpr int MNT = 64 * MWM * MWN;               // 512 threads
constexpr int MTM = MTB / MWM, MTN = NTB / MWN;   // 4 x 2 MFMA tiles per wave
static_assert(MTB * 64 == MNT && NTB * 64 == MNT, "one A and one B 16-byte slot per thread and stage");

typedef int v8i __attribute__((ext_vector_type(8)));

// e8m0 byte of a block's absmax: floor(log2 amax) is the fp32 exponent
// field minus 127 for a normal amax; a subnormal amax gives byte 0 (clamp)
__device__ __forceinline__ int mx_scale_byte(float amax) {
  if (amax == 0.0f) return 127;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return e - 2 < 0 ? 0 : e - 2;
}

// e2m1 code (0..15) of v = x / 2^X: nearest magnitude, ties to the even
// mantissa, saturating at 6
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float m = fabsf(v);
  float q;
  if (m < 2.0f) q = __builtin_rintf(m * 2.0f) * 0.5f;
  else if (m < 4.0f) q = __builtin_rintf(m);
  else q = __builtin_rintf(m * 0.5f) * 2.0f;
  q = fminf(q, 6.0f);
  const uint32_t idx = q < 2.0f ? (uint32_t)(q * 2.0f) : (q < 4.0f ? (uint32_t)q + 2u : (uint32_t)(q * 0.5f) + 4u);
  return idx | ((v < 0.0f && q > 0.0f) ? 8u : 0u);
}

// 32 values -> 16 bytes of codes (four dwords) and the scale byte
__device__ __forceinline__ int mx_block(const float (&x)[32], v4u &packed) {
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
  const int sb = mx_scale_byte(amax);
  const float inv = __int_as_float((254 - sb) << 23);   // 2^-(sb - 127), normal for sb in [0, 253]
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t d = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) d |= e2m1_code(x[8 * w + e] * inv) << (4 * e);
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

__global__ void k_mx_invlam(const uint16_t *lam, int K, float *inv) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k < K) inv[k] = 1.0f / f16_to_f32(lam[k]);
}

// Activations of one 16-row tile: thread t takes row t % 16 and the
// 32-blocks t / 16, t / 16 + 16, ...; its share of U (its blocks, in
// order) is summed over the 16 threads of its row in order through LDS.
template <int RP>
__global__ __launch_bounds__(256) void k_mx_quant(MxArgs a) {
  __shared__ float us[16][16][RP > 0 ? RP : 1];
  const int tid = threadIdx.x, row = tid & 15, q = tid >> 4;
  const int mt = blockIdx.x, m = mt * 16 + row;
  const int nb = 4 * a.KS;                        // 32-blocks incl. the pad of the last k-step
  float u[RP > 0 ? RP : 1];
#pragma unroll
  for (int c = 0; c < (RP > 0 ? RP : 1); ++c) u[c] = 0.0f;
  for (int b = q; b < nb; b += 16) {
    float x[32];
    const bool live = m < a.M && 32 * b < a.K;
    if (live) {
      const v4u *src = reinterpret_cast<const v4u *>(a.X + (size_t)m * a.K + 32 * b);
      const v4f *il = reinterpret_cast<const v4f *>(a.invlam + 32 * b);
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
    if constexpr (RP > 0) {
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
      if (c < a.r) a.U[(size_t)c * a.Mpad + mt * 16 + rr] = s;
    }
  }
}

template <int V>
struct int_c {
  static constexpr int value = V;
};

// The residual contraction with the epilogue: 8 waves in 2 x 4, each 64 x
// 32 outputs (4 x 2 MFMA tiles); one k-step (128 channels) per stage, two
// LDS buffers, the next stage's operands loaded into registers one stage
// ahead; scales straight from memory, one dword per tile and lane for four
// k-steps (byte j picked by a shift).
template <int RPT>
__global__ __launch_bounds__(MNT, 2) void k_mx_gemm(MxArgs a) {
  __shared__ alignas(16) uint8_t sa_[2][MTB][64][16];
  __shared__ alignas(16) uint8_t sb_[2][NTB][64][16];
  __shared__ float eu[RPT > 0 ? RPT : 1][MB];
  __shared__ float el2[RPT > 0 ? RPT : 1][NB];
  __shared__ float ebias[NB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / MWN, wn = wave % MWN;
  const int nblk = (a.N + NB - 1) / NB;
  const int mb = blockIdx.x / nblk, nb = blockIdx.x % nblk;
  const int mt0 = mb * MTB, nt0 = nb * NTB;
  const int MT = a.Mpad / 16, NT = (a.N + 15) / 16;
  const int KS = a.KS, KS4 = a.KS4;
  // operand slot of this thread: tile tid / 64, lane tid % 64
  const int tA = min(mt0 + (tid >> 6), MT - 1), tB = min(nt0 + (tid >> 6), NT - 1);
  const v4u *gA = reinterpret_cast<const v4u *>(a.qa) + ((size_t)tA * KS) * 64 + lane;
  const v4u *gB = reinterpret_cast<const v4u *>(a.wq) + ((size_t)tB * KS) * 64 + lane;
  // scale dwords of this lane's tiles
  const uint32_t *sA = reinterpret_cast<const uint32_t *>(a.sa);
  const uint32_t *sB = reinterpret_cast<const uint32_t *>(a.ws);

  // epilogue operands
  for (int p = tid; p < RPT * MB; p += MNT) {
    const int c = p / MB, rr = p % MB, m = mt0 * 16 + rr;
    eu[c][rr] = (c < a.r && m < a.M) ? a.U[(size_t)c * a.Mpad + m] : 0.0f;
  }
  for (int p = tid; p < RPT * NB; p += MNT) {
    const int c = p / NB, cc = p % NB, n = nt0 * 16 + cc;
    el2[c][cc] = (c < a.r && n < a.N) ? bf16_to_f32(a.L2[(size_t)c * a.N + n]) : 0.0f;
  }
  if (tid < NB) {
    const int n = nt0 * 16 + tid;
    ebias[tid] = (a.bias && n < a.N) ? bf16_to_f32(a.bias[n]) : 0.0f;
  }

  v4f acc[MTM][MTN];
#pragma unroll
  for (int i = 0; i < MTM; ++i)
#pragma unroll
    for (int j = 0; j < MTN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  v4u ra = gA[0], rb = gB[0];
  *reinterpret_cast<v4u *>(&sa_[0][tid >> 6][lane][0]) = ra;
  *reinterpret_cast<v4u *>(&sb_[0][tid >> 6][lane][0]) = rb;
  __syncthreads();

  uint32_t scA[MTM], scB[MTN];
  auto stage = [&](int ks, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;          // byte of the scale dwords
    const int buf = ks & 1;
    if (J == 0) {
#pragma unroll
      for (int i = 0; i < MTM; ++i)
        scA[i] = sA[(((size_t)min(mt0 + wm * MTM + i, MT - 1) * KS4 + (ks >> 2)) * 64 + lane)];
#pragma unroll
      for (int j = 0; j < MTN; ++j)
        scB[j] = sB[(((size_t)min(nt0 + wn * MTN + j, NT - 1) * KS4 + (ks >> 2)) * 64 + lane)];
    }
    if (ks + 1 < KS) {
      ra = gA[(size_t)(ks + 1) * 64];
      rb = gB[(size_t)(ks + 1) * 64];
    }
    v8i av[MTM], bv[MTN];
#pragma unroll
    for (int i = 0; i < MTM; ++i) {
      const v4u v = *reinterpret_cast<const v4u *>(&sa_[buf][wm * MTM + i][lane][0]);
      av[i] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < MTN; ++j) {
      const v4u v = *reinterpret_cast<const v4u *>(&sb_[buf][wn * MTN + j][lane][0]);
      bv[j] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < MTM; ++i)
#pragma unroll
      for (int j = 0; j < MTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av[i], bv[j], acc[i][j], 4, 4, 0, (int)((scA[i] >> (8 * J)) & 0xFFu), 0,
            (int)((scB[j] >> (8 * J)) & 0xFFu));
    if (ks + 1 < KS) {
      *reinterpret_cast<v4u *>(&sa_[buf ^ 1][tid >> 6][lane][0]) = ra;
      *reinterpret_cast<v4u *>(&sb_[buf ^ 1][tid >> 6][lane][0]) = rb;
    }
    __syncthreads();
  };
  int ks = 0;
  for (; ks + 4 <= KS; ks += 4) {
    stage(ks, int_c<0>{});
    stage(ks + 1, int_c<1>{});
    stage(ks + 2, int_c<2>{});
    stage(ks + 3, int_c<3>{});
  }
  if (ks < KS) stage(ks, int_c<0>{});
  if (ks + 1 < KS) stage(ks + 1, int_c<1>{});
  if (ks + 2 < KS) stage(ks + 2, int_c<2>{});

  // epilogue: Y = acc + U L2 + bias
  const int rowq = 4 * (lane >> 4), colq = lane & 15;
#pragma unroll
  for (int i = 0; i < MTM; ++i)
#pragma unroll
    for (int j = 0; j < MTN; ++j) {
      const int cc = (wn * MTN + j) * 16 + colq, n = nt0 * 16 + cc;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int rr = (wm * MTM + i) * 16 + rowq + qq, m = mt0 * 16 + rr;
        float y = acc[i][j][qq];
#pragma unroll
        for (int c = 0; c < RPT; ++c) y = __builtin_fmaf(eu[c][rr], el2[c][cc], y);
        y += ebias[cc];
        if (m < a.M && n < a.N) {
          const size_t off = (size_t)m * a.N + n;
          if (a.y_bf16)
            reinterpret_cast<uint16_t *>(a.Y)[off] = f32_to_bf16(y);
          else
            reinterpret_cast<float *>(a.Y)[off] = y;
        }
      }
    }
}

template <int RP>
hipError_t launch_mx_rp(const MxArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_mx_quant<RP>, dim3((unsigned)(a.Mpad / 16)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tiles = ceil_div(a.N, NB) * ceil_div(a.M, MB);
  hipLaunchKernelGGL(k_mx_gemm<RP>, dim3((unsigned)tiles), dim3(MNT), 0, s, a);
  return hipGetLastError();
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
  L.invlam_off = off;
  off = align_up(off + (size_t)K * sizeof(float), 256);
  L.qa_off = off;
  off = align_up(off + (size_t)(L.Mpad / 16) * L.KS * 1024, 256);
  L.sa_off = off;
  off = align_up(off + (size_t)(L.Mpad / 16) * L.KS4 * 256, 256);
  L.u_off = off;
  off = align_up(off + (size_t)r * L.Mpad * sizeof(float), 256);
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
  hipLaunchKernelGGL(k_mx_invlam, dim3((unsigned)ceil_div(a.K, 256)), dim3(256), 0, s, a.lam, a.K, a.invlam);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.r == 0) return launch_mx_rp<0>(a, s);
  if (a.r <= 4) return launch_mx_rp<4>(a, s);
  if (a.r <= 8) return launch_mx_rp<8>(a, s);
  if (a.r <= 16) return launch_mx_rp<16>(a, s);
  return launch_mx_rp<32>(a, s);
}

}  // namespace hsq

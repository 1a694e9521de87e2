// calib.hip -- the calibration steps of the method on the GPU: the Hessian
// H = Xh^T Xh of the smoothed calibration activations, its deflation by the
// protected subspace span(L1), and the closed-form output-side factor L2.
//
// Method (Deflating the Hessian, paper page: abstract and Figure 1
// caption; H-SVDQuant explainer, rit.work, section on Hessian deflation):
// for a fixed input-side factor L1 (K x r) the output-side factor is
// eliminated in closed form, L2* = C^-1 L1^T H E with C = L1^T H L1 and
// E = W - deq(Q(R)), which leaves the deflated Hessian
// Hperp = H - H L1 C^-1 L1^T H (Hperp L1 = 0) as the metric of the residual.
//
// Kernels:
//   k_hessian   bf16 MFMA (16x16x32) over the token dimension: one 128 x 128
//               block of H per workgroup, upper-triangle blocks only, the
//               mirror written by the same workgroup.  X is row-major
//               (token x channel), so the operand tiles are transposed on
//               the way into LDS (channel-major, tokens contiguous).  The
//               products of bf16 inputs are exact in fp32; the smoothing
//               1/lambda multiplies the finished sums, row and column.
//               Few blocks (small K): the tokens are split across
//               workgroups, with fp32 partial blocks summed in split order.
//   k_hl1       H L1 (K x r) row by row, one wave per row, reading H once;
//               each workgroup also sums its rows' share of C = L1^T H L1 in
//               fp64.
//   k_cinv      C from the workgroup shares (fixed order, fp64) and its
//               inverse by Gauss-Jordan elimination with partial pivoting,
//               in one workgroup (r <= 32).
//   k_deflate   Hperp = H - B HL1^T with B = HL1 C^-1: a rank-r update,
//               HBM-bound (H read once, Hperp written once; may be in place).
//   k_l2_part / k_l2_final
//               T = HL1^T E over K slices (E decoded on the fly from W, the
//               packed residual codes and their scales), then L2 = C^-1 T.
#include "hsq_internal.h"

#include <algorithm>

namespace hsq {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- Hessian
constexpr int HB = 128;            // block of H (rows = columns)
constexpr int HKC = 64;            // tokens per stage
constexpr int HNT = 512;           // threads: 8 waves, 2 x 4, 64 x 32 each
constexpr int kHessFull = 0, kHessSplit = 1, kHessReduce = 2;
constexpr int HTM = 4, HTN = 2;    // 16 x 16 tiles per wave
constexpr int kHessAcc = HTM * HTN * 4;  // accumulators per thread

struct alignas(16) HessSmem {
  uint16_t t[2][2][HKC][HB];       // [buffer][row, column strip][token in stage][channel, swizzled]
};

// Swizzle of a token row's sixteen 16-byte chunks (eight channels each):
// logical chunk c sits at c ^ hess_swz(t).  The transposing reads of a k-step
// touch four consecutive token rows and two adjacent chunks per 16-lane
// group; with this even XOR the 32 lanes of two groups (tokens t .. t + 3 and
// t + 8 .. t + 11) reach 16 distinct chunk positions.
__device__ __forceinline__ int hess_swz(int t) { return 2 * ((t & 3) | (((t >> 3) & 1) << 2)); }

constexpr int kSuper = 8;          // blocks per side of a super-block

// workgroup id -> (row block, column block), bi <= bj.  Consecutive ids go
// to different XCDs (id % 8), each with its own L2; regroup them so that
// XCD x owns a contiguous range of an order that walks the upper triangle
// in kSuper x kSuper super-blocks (row-major over super-blocks, row-major
// inside).  The workgroups an XCD runs at once then share a few row and
// column strips of X per stage instead of touching every strip.
__device__ __forceinline__ void hess_block(int bid, int nb, int &bi, int &bj) {
  const int T = nb * (nb + 1) / 2;
  const int per = T / 8, rem = T % 8, x = bid % 8, loc = bid / 8;
  int t = x * per + min(x, rem) + loc;
  const int nsb = (nb + kSuper - 1) / kSuper;
  for (int I = 0; I < nsb; ++I) {
    const int rows = min(kSuper, nb - I * kSuper);
    for (int J = I; J < nsb; ++J) {
      const int cols = min(kSuper, nb - J * kSuper);
      const int cnt = I == J ? rows * (rows + 1) / 2 : rows * cols;
      if (t < cnt) {
        if (I != J) {
          bi = I * kSuper + t / cols;
          bj = J * kSuper + t % cols;
        } else {
          int i = 0, len = rows;
          while (t >= len) {
            t -= len;
            ++i;
            --len;
          }
          bi = I * kSuper + i;
          bj = I * kSuper + i + t;
        }
        return;
      }
      t -= cnt;
    }
  }
  bi = bj = 0;                    // unreachable: bid < T
}

template <int MODE>
__global__ __launch_bounds__(HNT, 2) void k_hessian(HessArgs a) {
  __shared__ HessSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 2, wc = wave & 3;
  const int nb = (a.K + HB - 1) / HB;
  int bi, bj;
  hess_block(blockIdx.x, nb, bi, bj);
  const bool diag = bi == bj;
  const int I0 = bi * HB, J0 = bj * HB;
  const int nblk = nb * (nb + 1) / 2;
  // partial blocks: [split][block][chunk][thread] float4
  float *part = a.part + ((size_t)blockIdx.y * nblk + blockIdx.x) * (HNT * kHessAcc);

  float acc[HTM][HTN][4];
#pragma unroll
  for (int i = 0; i < HTM; ++i)
#pragma unroll
    for (int j = 0; j < HTN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][j][q] = 0.0f;

  if constexpr (MODE != kHessReduce) {
    // token range of this split, whole stages
    const int nst = (a.M + HKC - 1) / HKC, S = (int)gridDim.y, z = (int)blockIdx.y;
    const int s0 = z * nst / S, s1 = (z + 1) * nst / S;
    const int m_end = min(a.M, s1 * HKC);
    // Stage loads: waves 0-3 move the row strip (channels I0 ..), waves 4-7
    // the column strip (J0 ..); wave w's four direct-to-LDS loads cover
    // token rows 16 (w % 4) .. + 15 of the stage, four rows (1 KB) each.
    // Lane l of a load fills token row 4d + l / 16 at physical chunk l % 16,
    // i.e. logical chunk (l % 16) ^ hess_swz(row): the channels 8c .. 8c + 7
    // of that token.  Tokens past the split's end and channels past K read
    // zero (an offset past the buffer).
    const v4u rx = raw_rsrc(a.X, (uint32_t)((size_t)a.M * a.K * 2));
    const uint32_t kBad = 0x80000000u;
    const int strip = wave >> 2, d0 = 4 * (wave & 3);
    const int trow = lane >> 4;                             // token row within a load
    const int cbase = strip ? J0 : I0;
    auto issue = [&](int s, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = 4 * (d0 + u) + trow, m = s * HKC + t;
        const int ch = cbase + 8 * ((lane & 15) ^ hess_swz(t));
        const uint32_t off = (m < m_end && ch < a.K) ? ((uint32_t)m * (uint32_t)a.K + (uint32_t)ch) * 2u : kBad;
        block_to_lds(rx, lds_addr(&sm.t[buf][strip][4 * (d0 + u)][0]), off, 0u);
      }
    };
    // Operand reads: the MFMA's lane l takes channel (tile base) + l % 16 and
    // tokens 8 (l / 16) .. + 7 of the k-step.  ds_read_b64_tr_b16 gives lane
    // i of each 16-lane group element j = the 16-bit value at element i % 4
    // of the 8 bytes that lane 4 j + i / 4 of the group addressed; so lane
    // L = 4 jt + q addresses token jt (of four) and channels 4 q .. 4 q + 3,
    // and two reads (tokens 0-3, then 4-7) give the eight values.  The
    // swizzle of a token row depends only on jt and bit 3 of the token, both
    // fixed per lane, so each tile's byte offset is fixed per lane.
    const int g = lane >> 4, L = lane & 15, jt = L >> 2, q = L & 3;
    const int sw = hess_swz(8 * g + jt);                    // = the swizzle of every token this lane reads
    uint32_t offa[HTM], offb[HTN];
#pragma unroll
    for (int i = 0; i < HTM; ++i) {
      const int c = (64 * wr + 16 * i) / 8 + (q >> 1);
      offa[i] = (uint32_t)((8 * g + jt) * HB * 2 + ((c ^ sw) * 16) + (q & 1) * 8);
    }
#pragma unroll
    for (int j = 0; j < HTN; ++j) {
      const int c = (32 * wc + 16 * j) / 8 + (q >> 1);
      offb[j] = (uint32_t)((8 * g + jt) * HB * 2 + ((c ^ sw) * 16) + (q & 1) * 8);
    }
    auto rd = [&](int buf, int st, uint32_t off) __attribute__((always_inline)) -> v4s {
      const char *p = reinterpret_cast<const char *>(&sm.t[buf][st][0][0]) + off;
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
    };
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        constexpr uint32_t kRow4 = 4 * HB * 2;               // four token rows
        const uint32_t kofs = (uint32_t)kk * 32 * HB * 2;   // the k-step's 32 token rows
        v8bf av[HTM], bv[HTN];
#pragma unroll
        for (int i = 0; i < HTM; ++i) {
          const v4s lo = rd(buf, 0, offa[i] + kofs), hi = rd(buf, 0, offa[i] + kofs + kRow4);
          av[i] = __builtin_bit_cast(v8bf, (v8s){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
#pragma unroll
        for (int j = 0; j < HTN; ++j) {
          const v4s lo = rd(buf, 1, offb[j] + kofs), hi = rd(buf, 1, offb[j] + kofs + kRow4);
          bv[j] = __builtin_bit_cast(v8bf, (v8s){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
#pragma unroll
        for (int i = 0; i < HTM; ++i)
#pragma unroll
          for (int j = 0; j < HTN; ++j) {
            v4f c4 = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], c4, 0, 0, 0);
            acc[i][j][0] = c4[0]; acc[i][j][1] = c4[1]; acc[i][j][2] = c4[2]; acc[i][j][3] = c4[3];
          }
      }
    };
    // one stage ahead in the other buffer; stage_barrier waits for this
    // wave's loads and LDS reads, then the workgroup
    if (s0 < s1) issue(s0, 0);
    stage_barrier();
    for (int s = s0; s < s1; ++s) {
      const int buf = (s - s0) & 1;
      if (s + 1 < s1) issue(s + 1, buf ^ 1);
      compute(buf);
      stage_barrier();
    }
  }

  if constexpr (MODE == kHessSplit) {
#pragma unroll
    for (int i = 0; i < HTM; ++i)
#pragma unroll
      for (int j = 0; j < HTN; ++j)
        *reinterpret_cast<v4f *>(part + ((i * HTN + j) * HNT + tid) * 4) =
            (v4f){acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
    return;
  } else {
    if constexpr (MODE == kHessReduce) {
      // the partial blocks in split order
      for (int z = 0; z < a.splits; ++z) {
        const float *src = a.part + ((size_t)z * nblk + blockIdx.x) * (HNT * kHessAcc);
#pragma unroll
        for (int i = 0; i < HTM; ++i)
#pragma unroll
          for (int j = 0; j < HTN; ++j) {
            const v4f v = *reinterpret_cast<const v4f *>(src + ((i * HTN + j) * HNT + tid) * 4);
            acc[i][j][0] += v[0]; acc[i][j][1] += v[1]; acc[i][j][2] += v[2]; acc[i][j][3] += v[3];
          }
      }
    }
    // H[i][j] (+)= fl(S * fl(d_i * d_j)), d = fl32(1 / lambda): symmetric
    // in (i, j), so the two triangles of a diagonal block (computed apart)
    // agree bit for bit; the mirror of an off-diagonal block gets the same
    // values transposed (four consecutive columns of one row per lane: one
    // 16-byte store)
#pragma unroll
    for (int i = 0; i < HTM; ++i) {
      const int gi0 = I0 + 64 * wr + 16 * i + 4 * (lane >> 4);   // rows gi0 .. gi0 + 3
      if (gi0 >= a.K) continue;
      float di[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) di[q] = 1.0f / f16_to_f32(a.lam[gi0 + q]);
#pragma unroll
      for (int j = 0; j < HTN; ++j) {
        const int gj = J0 + 32 * wc + 16 * j + (lane & 15);
        if (gj >= a.K) continue;
        const float dj = 1.0f / f16_to_f32(a.lam[gj]);
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[i][j][q] * (di[q] * dj);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float *h = a.H + (size_t)(gi0 + q) * a.K + gj;
          *h = a.accumulate ? *h + v[q] : v[q];
        }
        if (!diag) {
          v4f *h = reinterpret_cast<v4f *>(a.H + (size_t)gj * a.K + gi0);
          v4f o = (v4f){v[0], v[1], v[2], v[3]};
          if (a.accumulate) o += *h;
          *h = o;
        }
      }
    }
  }
}

int hess_blocks(int K) {
  const int nb = ceil_div(K, HB);
  return nb * (nb + 1) / 2;
}

}  // namespace

// Token splits of the Hessian: enough workgroups for two per CU, each
// split at least 4 stages (256 tokens), at most 16 splits.
int hessian_splits(int M, int K) {
  const int blocks = hess_blocks(K), stages = ceil_div(M, HKC);
  int S = ceil_div(2 * 256, blocks);
  S = std::min(S, std::max(1, stages / 4));
  return std::max(1, std::min(S, 16));
}

size_t hessian_workspace_bytes(int M, int K) {
  const int S = hessian_splits(M, K);
  return S > 1 ? (size_t)S * hess_blocks(K) * HNT * kHessAcc * sizeof(float) : 0;
}

hipError_t launch_hessian(const HessArgs &a0, hipStream_t s) {
  HessArgs a = a0;
  a.splits = hessian_splits(a.M, a.K);
  const unsigned blocks = (unsigned)hess_blocks(a.K);
  if (a.splits <= 1) {
    hipLaunchKernelGGL(k_hessian<kHessFull>, dim3(blocks, 1u), dim3(HNT), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_hessian<kHessSplit>, dim3(blocks, (unsigned)a.splits), dim3(HNT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hessian<kHessReduce>, dim3(blocks, 1u), dim3(HNT), 0, s, a);
  return hipGetLastError();
}

namespace {

// ---------------------------------------------------------------- deflation
constexpr int DNT = 256;           // threads of the deflation kernels
constexpr int kHl1Waves = DNT / 64;
constexpr int kHl1MaxWgs = 1024;
constexpr int kDefRows = 16;       // rows of H per deflation workgroup
constexpr int kDefCols = 4 * DNT;  // columns per deflation workgroup

// L1 (bf16, K x r) as fp32 rows padded to RP (zeros past r)
template <int RP>
__global__ void k_l1f(const uint16_t *L1, int K, int r, float *L1f) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= K * RP) return;
  const int k = i / RP, c = i % RP;
  L1f[i] = c < r ? bf16_to_f32(L1[(size_t)k * r + c]) : 0.0f;
}

// one wave per row of H: HL1[i][:] = sum_k H[i][k] L1[k][:], lanes over k in
// 16-byte chunks; the wave's rows also add L1[i][a] * HL1[i][b] into the
// workgroup's share of C (fp64, rows in order, waves in order)
template <int RP>
__global__ __launch_bounds__(DNT) void k_hl1(DeflArgs a) {
  __shared__ double cs[kHl1Waves][RP * RP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int CPL = (RP * RP + 63) / 64;          // C entries per lane
  double cp[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) cp[e] = 0.0;
  const int nw = gridDim.x * kHl1Waves;
  for (int i = blockIdx.x * kHl1Waves + wave; i < a.K; i += nw) {
    const float *hrow = a.H + (size_t)i * a.K;
    float acc[RP];
#pragma unroll
    for (int c = 0; c < RP; ++c) acc[c] = 0.0f;
    for (int k = 4 * lane; k < a.K; k += 256) {
      const v4f h = *reinterpret_cast<const v4f *>(hrow + k);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float *l = a.L1f + (size_t)(k + u) * RP;
#pragma unroll
        for (int c = 0; c < RP; c += 4) {
          const v4f l4 = *reinterpret_cast<const v4f *>(l + c);
          acc[c] = __builtin_fmaf(h[u], l4[0], acc[c]);
          acc[c + 1] = __builtin_fmaf(h[u], l4[1], acc[c + 1]);
          acc[c + 2] = __builtin_fmaf(h[u], l4[2], acc[c + 2]);
          acc[c + 3] = __builtin_fmaf(h[u], l4[3], acc[c + 3]);
        }
      }
    }
    // butterfly: every lane ends with the row's totals (same order in all lanes)
#pragma unroll
    for (int c = 0; c < RP; ++c) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc[c] += __shfl_xor(acc[c], o, 64);
    }
    if (lane < a.r) {
      float v = acc[0];
#pragma unroll
      for (int c = 1; c < RP; ++c)
        if (lane == c) v = acc[c];
      a.HL1[(size_t)i * a.r + lane] = v;
    }
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int p = lane + 64 * e;
      if (p < RP * RP) {
        const int ca = p / RP, cb = p % RP;
        float hb = acc[0];
#pragma unroll
        for (int c = 1; c < RP; ++c)
          if (cb == c) hb = acc[c];
        cp[e] += (double)a.L1f[(size_t)i * RP + ca] * (double)hb;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const int p = lane + 64 * e;
    if (p < RP * RP) cs[wave][p] = cp[e];
  }
  __syncthreads();
  for (int p = tid; p < RP * RP; p += DNT) {
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kHl1Waves; ++w) v += cs[w][p];
    a.Cpart[(size_t)p * gridDim.x + blockIdx.x] = v;   // entry-major: the sum reads rows
  }
}

// C = sum of the workgroup shares (in order), then C^-1 by Gauss-Jordan
// elimination with partial pivoting on [C | I] in fp64.  A singular C
// (pivot exactly 0) yields NaN in C^-1.
template <int RP>
__global__ __launch_bounds__(DNT) void k_cinv(DeflArgs a, int nparts) {
  __shared__ double m[RP][2 * RP];
  __shared__ double f[RP];
  __shared__ int piv;
  const int tid = threadIdx.x, r = a.r, lane = tid & 63, wave = tid >> 6;
  // entry p of C by wave p % 4: lane l adds shares l, l + 64, ... in order,
  // then a butterfly over the lanes (the same order in every lane)
  for (int p = wave; p < RP * RP; p += DNT / 64) {
    double v = 0.0;
#pragma unroll 16
    for (int w = lane; w < nparts; w += 64) v += a.Cpart[(size_t)p * nparts + w];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) m[p / RP][p % RP] = v;
  }
  for (int p = tid; p < RP * RP; p += DNT) m[p / RP][RP + p % RP] = (p / RP == p % RP) ? 1.0 : 0.0;
  __syncthreads();
  for (int c = 0; c < r; ++c) {
    if (tid == 0) {
      int p = c;
      for (int i = c + 1; i < r; ++i)
        if (fabs(m[i][c]) > fabs(m[p][c])) p = i;
      piv = p;
    }
    __syncthreads();
    const int p = piv;
    if (p != c)
      for (int j = tid; j < 2 * RP; j += DNT) {
        const double t = m[c][j];
        m[c][j] = m[p][j];
        m[p][j] = t;
      }
    __syncthreads();
    const double d = m[c][c];
    __syncthreads();
    for (int j = tid; j < 2 * RP; j += DNT) m[c][j] = d != 0.0 ? m[c][j] / d : __builtin_nan("");
    for (int i = tid; i < RP; i += DNT) f[i] = m[i][c];
    __syncthreads();
    for (int e = tid; e < RP * 2 * RP; e += DNT) {
      const int i = e / (2 * RP), j = e % (2 * RP);
      if (i != c && i < r) m[i][j] = __builtin_fma(-f[i], m[c][j], m[i][j]);
    }
    __syncthreads();
  }
  for (int p = tid; p < r * r; p += DNT) a.Cinv[p] = m[p / r][RP + p % r];
}

// Hperp[i][j] = H[i][j] - sum_a B[i][a] HL1[j][a], B = HL1 C^-1.  A thread
// owns four adjacent columns (their HL1 rows in registers) and walks the
// workgroup's kDefRows rows.
template <int RP>
__global__ __launch_bounds__(DNT) void k_deflate(DeflArgs a) {
  __shared__ float bs[kDefRows][RP];
  __shared__ double ci[RP * RP];
  const int tid = threadIdx.x, r = a.r;
  const int j0 = blockIdx.x * kDefCols + 4 * tid;
  const int i0 = blockIdx.y * kDefRows;
  for (int p = tid; p < r * r; p += DNT) ci[p] = a.Cinv[p];
  float hl[4][RP];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int c = 0; c < RP; ++c)
      hl[u][c] = (c < r && j0 + u < a.K) ? a.HL1[(size_t)(j0 + u) * r + c] : 0.0f;
  __syncthreads();
  for (int p = tid; p < kDefRows * RP; p += DNT) {
    const int ii = p / RP, c = p % RP, i = i0 + ii;
    double v = 0.0;
    if (c < r && i < a.K)
      for (int b = 0; b < r; ++b) v += (double)a.HL1[(size_t)i * r + b] * ci[b * r + c];
    bs[ii][c] = (float)v;
  }
  __syncthreads();
  if (j0 >= a.K) return;
  for (int ii = 0; ii < kDefRows; ++ii) {
    const int i = i0 + ii;
    if (i >= a.K) break;
    v4f h = *reinterpret_cast<const v4f *>(a.H + (size_t)i * a.K + j0);
#pragma unroll
    for (int c = 0; c < RP; ++c) {
      const float b = bs[ii][c];
#pragma unroll
      for (int u = 0; u < 4; ++u) h[u] = __builtin_fmaf(-b, hl[u][c], h[u]);
    }
    *reinterpret_cast<v4f *>(a.Hperp + (size_t)i * a.K + j0) = h;
  }
}

// ---------------------------------------------------------------- closed-form L2
constexpr int LNT = 256;           // threads (= columns) per workgroup

// T_s[c][n] = sum over the slice's channels k of HL1[k][c] * E[k][n],
// E = W - code * sw.  A thread owns column n; the slice's HL1 rows sit in
// LDS (read as broadcasts).
template <int RP>
__global__ __launch_bounds__(LNT) void k_l2_part(L2Args a) {
  extern __shared__ float hl[];                 // [channels of the slice][RP]
  const int tid = threadIdx.x;
  const int n = blockIdx.x * LNT + tid;
  const int nblk64 = a.K / kGroup, S = (int)gridDim.y, z = (int)blockIdx.y;
  const int b0 = z * nblk64 / S, b1 = (z + 1) * nblk64 / S;   // 64-channel blocks of the slice
  const int k0 = b0 * kGroup, kn = (b1 - b0) * kGroup;
  for (int p = tid; p < kn * RP; p += LNT) {
    const int kk = p / RP, c = p % RP;
    hl[p] = c < a.r ? a.HL1[(size_t)(k0 + kk) * a.r + c] : 0.0f;
  }
  __syncthreads();
  if (n >= a.N) return;
  const int GP = (a.K / kGroup + 1) / 2, nt = n >> 4;      // group pairs of the packed blob
  float t[RP];
#pragma unroll
  for (int c = 0; c < RP; ++c) t[c] = 0.0f;
  for (int b = b0; b < b1; ++b) {
    const float s = f16_to_f32(a.sw[(size_t)(b * kGroup / a.group) * a.N + n]);
    const uint8_t *blk = a.packed + ((size_t)nt * GP + (b >> 1)) * 1024 + 8 * (b & 1);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const v2u w = *reinterpret_cast<const v2u *>(blk + ((n & 15) + 16 * kq) * 16);
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        // nibble of channel p (two's complement): bytes 0-3 of the first
        // dword hold p = 0-3 (high nibbles) and 4-7 (low); the second
        // dword p = 8-11 (high) and 12-15 (low)
        const uint32_t word = p < 8 ? w.x : w.y;
        const int pb = p & 7;
        const int sh = pb < 4 ? 8 * pb + 4 : 8 * (pb - 4);
        const int code = __builtin_amdgcn_sbfe((int)word, sh, 4);
        const int k = b * kGroup + 16 * kq + p;
        const float wv = bf16_to_f32(a.W[(size_t)k * a.N + n]);
        const float e = __builtin_fmaf(-(float)code, s, wv);
        const float *h = hl + (size_t)(k - k0) * RP;
#pragma unroll
        for (int c = 0; c < RP; ++c) t[c] = __builtin_fmaf(h[c], e, t[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < RP; ++c)
    if (c < a.r) a.Tpart[((size_t)z * a.r + c) * a.N + n] = t[c];
}

// L2[c][n] = sum_b C^-1[c][b] * sum_s T_s[b][n] (slices in order, fp64).
// Thread (column, rank row b) sums T_s[b][n] over the slices; the
// workgroup's columns then meet in LDS for the r x r product.
template <int RP>
__global__ __launch_bounds__(LNT) void k_l2_final(L2Args a, int S) {
  constexpr int CPW = LNT / RP;                   // columns per workgroup
  __shared__ double tb[RP][CPW];
  const int b = threadIdx.x / CPW, cl = threadIdx.x % CPW;
  const int n = blockIdx.x * CPW + cl;
  double v = 0.0;
  if (b < a.r && n < a.N) {
    const float *src = a.Tpart + (size_t)b * a.N + n;
#pragma unroll 8
    for (int z = 0; z < S; ++z) v += (double)src[(size_t)z * a.r * a.N];
  }
  tb[b][cl] = v;
  __syncthreads();
  const int c = b;
  if (c < a.r && n < a.N) {
    double y = 0.0;
    for (int k = 0; k < a.r; ++k) y += a.Cinv[c * a.r + k] * tb[k][cl];
    a.L2[(size_t)c * a.N + n] = (float)y;
  }
}

template <int RP>
hipError_t launch_defl_rp(const DeflArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_l1f<RP>, dim3((unsigned)ceil_div(a.K * RP, 256)), dim3(256), 0, s, a.L1, a.K, a.r,
                     a.L1f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int wgs = deflate_hl1_wgs(a.K);
  hipLaunchKernelGGL(k_hl1<RP>, dim3((unsigned)wgs), dim3(DNT), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_cinv<RP>, dim3(1), dim3(DNT), 0, s, a, wgs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_deflate<RP>, dim3((unsigned)ceil_div(a.K, kDefCols), (unsigned)ceil_div(a.K, kDefRows)),
                     dim3(DNT), 0, s, a);
  return hipGetLastError();
}

template <int RP>
hipError_t launch_l2_rp(const L2Args &a, hipStream_t s) {
  const int S = l2_slices(a.K, a.N, a.r);
  const int ch = a.K / kGroup;                       // 64-channel blocks
  const int maxk = ceil_div(ch, S) * kGroup;         // channels of the longest slice
  hipLaunchKernelGGL(k_l2_part<RP>, dim3((unsigned)ceil_div(a.N, LNT), (unsigned)S), dim3(LNT),
                     (size_t)maxk * RP * sizeof(float), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_l2_final<RP>, dim3((unsigned)ceil_div(a.N, LNT / RP)), dim3(LNT), 0, s, a, S);
  return hipGetLastError();
}

}  // namespace

int deflate_hl1_wgs(int K) { return std::min(kHl1MaxWgs, ceil_div(K, kHl1Waves)); }

int rank_pad(int r) { return r <= 4 ? 4 : r <= 8 ? 8 : r <= 16 ? 16 : 32; }

size_t deflate_workspace_bytes(int K, int r) {
  const int RP = rank_pad(r);
  return align_up((size_t)K * RP * sizeof(float), 256) +
         (size_t)deflate_hl1_wgs(K) * RP * RP * sizeof(double);
}

hipError_t launch_deflate(const DeflArgs &a, hipStream_t s) {
  switch (rank_pad(a.r)) {
    case 4: return launch_defl_rp<4>(a, s);
    case 8: return launch_defl_rp<8>(a, s);
    case 16: return launch_defl_rp<16>(a, s);
    default: return launch_defl_rp<32>(a, s);
  }
}

// K slices of the L2 pass: about 2048 workgroups (8 per CU: each thread
// walks its column's channels one after the other, so the pass needs many
// waves in flight), at most one per 64-channel block, and enough that a
// slice's HL1 rows fit 64 KB of LDS (at most 256 / RP blocks per slice).
int l2_slices(int K, int N, int r) {
  const int cols = ceil_div(N, LNT), blocks = K / kGroup;
  const int S = std::max(ceil_div(2048, cols), ceil_div(blocks * rank_pad(r), 256));
  return std::max(1, std::min(S, blocks));
}

size_t l2_workspace_bytes(int K, int N, int r) {
  return (size_t)l2_slices(K, N, r) * r * N * sizeof(float);
}

hipError_t launch_l2(const L2Args &a, hipStream_t s) {
  switch (rank_pad(a.r)) {
    case 4: return launch_l2_rp<4>(a, s);
    case 8: return launch_l2_rp<8>(a, s);
    case 16: return launch_l2_rp<16>(a, s);
    default: return launch_l2_rp<32>(a, s);
  }
}

}  // namespace hsq

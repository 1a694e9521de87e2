// probe.hip -- measurement kernels (libhsq_probe, declared in hsq_probe.h):
// the int8 MFMA rate with and without the residual contraction's per-group
// rescale, and HBM streaming rates.  They measure the chip, not the method.
//
// The MFMA probe gives each wave the tiled contraction's wave tile (4 x 2
// MFMA tiles of 16x16) and step structure: MFMAs of row tile s, then the
// VALU work of row tile s-1 (a software pipeline over the four rows), all
// operands in registers, optionally with the loop's LDS operand reads.  Its
// rates are the ceilings the contraction is measured against.
#include "hsq_probe.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kMagicBits = 0x4B400000;   // bits of 1.5 * 2^23
constexpr int TM = 4;                    // MFMA row tiles per wave (64 rows)

__device__ __forceinline__ void pin(v4i &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

// LDS of the MODE 3 loop: the tiled contraction's stage buffers (two
// buffers of 8 A tiles and 8 B tiles of 64 lanes x 16 bytes, 128 weight
// scale pairs, 8 x 16 activation scales), read as its waves read them:
// wave (wm, wn) of the 2 x 4 arrangement reads A tiles 4wm..4wm+3 and B
// tiles 2wn, 2wn+1
struct alignas(16) StageLds {
  int8_t a[2][8][64][16];
  int8_t b[2][8][64][16];
  float2 sw[2][128];
  _Float16 sx[2][8][16];
};
constexpr int kMaxWaves = 16;

// the wide tile needs about 150 registers: at most 8 waves per workgroup
template <int MODE, int TN>
__global__ __launch_bounds__(TN == 4 ? 512 : 64 * kMaxWaves) void k_probe_mfma(int iters, float s0, int32_t *out) {
  __shared__ StageLds lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int colq = lane & 15, rowq = 4 * (lane >> 4);
  const v4i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};

  v4i a[TM], b[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a[i] = (v4i){lane + i, 3 * lane, 0x01010101 * (i + 1), -lane};
#pragma unroll
  for (int j = 0; j < TN; ++j) b[j] = (v4i){0x10101010 * (j + 1), lane, -3 * lane, 7};
  float2 sw[TN];
  v4h sx[TM];
#pragma unroll
  for (int j = 0; j < TN; ++j) sw[j] = make_float2(1.0f / 16.0f + lane * 1e-6f, -kMagicBits * 1e-9f);
#pragma unroll
  for (int i = 0; i < TM; ++i)       // run-time values: no constant folding of the rescale
    sx[i] = (v4h){(_Float16)s0, (_Float16)(s0 * 0.5f), (_Float16)(s0 * 0.25f), (_Float16)(s0 + lane)};

  const int wm = (wave >> 2) & 1, wn = wave & 3;
  if constexpr (MODE == 3) {
    for (int t = threadIdx.x; t < 2 * 8 * 64; t += blockDim.x) {
      const int bf = t >> 9, tile = (t >> 6) & 7, l = t & 63;
      *reinterpret_cast<v4i *>(&lds.a[bf][tile][l][0]) = (v4i){l, tile, bf, 0x01010101};
      *reinterpret_cast<v4i *>(&lds.b[bf][tile][l][0]) = (v4i){0x10101010, l, tile, bf};
    }
    for (int t = threadIdx.x; t < 2 * 128; t += blockDim.x) {
      lds.sw[t >> 7][t & 127] = sw[0];
      lds.sx[t >> 7][(t >> 4) & 7][t & 15] = (_Float16)1.0f;
    }
    __syncthreads();
  }

  v4i d[TM][TN];
  float acc[TM][TN][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      d[i][j] = magic;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][j][q] = 0.0f;
    }

  auto rescale = [&](int i) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (MODE == 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(__int_as_float(d[i][j][q]), sw[j].x, acc[i][j][q]);
      } else {
        const float u0 = __builtin_fmaf(__int_as_float(d[i][j][0]), sw[j].x, sw[j].y);
        const float u1 = __builtin_fmaf(__int_as_float(d[i][j][1]), sw[j].x, sw[j].y);
        const float u2 = __builtin_fmaf(__int_as_float(d[i][j][2]), sw[j].x, sw[j].y);
        const float u3 = __builtin_fmaf(__int_as_float(d[i][j][3]), sw[j].x, sw[j].y);
        acc[i][j][0] = __builtin_fmaf(u0, (float)sx[i].x, acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(u1, (float)sx[i].y, acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(u2, (float)sx[i].z, acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(u3, (float)sx[i].w, acc[i][j][3]);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) pin(acc[i][j][q]);
  };

  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 3) {
      // the step's operand reads, from the buffer of this step's parity
      const int bf = it & 1;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        b[j] = *reinterpret_cast<const v4i *>(&lds.b[bf][(wn * TN + j) & 7][lane][0]);
        sw[j] = lds.sw[bf][((wn * TN + j) & 7) * 16 + colq];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        a[i] = *reinterpret_cast<const v4i *>(&lds.a[bf][wm * TM + i][lane][0]);
        sx[i] = *reinterpret_cast<const v4h *>(&lds.sx[bf][wm * TM + i][rowq]);
      }
    }
#pragma unroll
    for (int s = 0; s < TM; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      pin(a[s]);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (MODE == 0)
          d[s][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[s], b[j], d[s][j], 0, 0, 0);
        else
          d[s][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[s], b[j], magic, 0, 0, 0);
      }
      if constexpr (MODE != 0) {
        rescale(s == 0 ? TM - 1 : s - 1);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, MODE == 1 ? 4 : 8, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  int sum = 0;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) sum ^= d[i][j][q] ^ __float_as_int(acc[i][j][q]);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kStreamThreads) void k_probe_read(const v4u *__restrict__ src, size_t n16,
                                                               int32_t *__restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  unsigned x = 0;
  size_t i = tid;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    v4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const v4u v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = (int32_t)x;
}

__global__ __launch_bounds__(kStreamThreads) void k_probe_copy(const v4u *__restrict__ src, size_t n16,
                                                               v4u *__restrict__ dst) {
  const size_t tid = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = tid;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    v4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int status(hipError_t e) { return e == hipSuccess ? 0 : -5; }

}  // namespace

extern "C" {

int hsq_probe_mfma(int mode, int iters, int blocks, int waves, int32_t *out, void *stream) {
  if (mode < 0 || mode > 5 || iters < 1 || blocks < 1 || waves < 1 || waves > (mode >= 4 ? 8 : kMaxWaves) || !out)
    return -1;
  if (!aligned16(out)) return -3;
  const dim3 grid((unsigned)blocks), block((unsigned)(64 * waves));
  hipStream_t s = (hipStream_t)stream;
  switch (mode) {
    case 0: hipLaunchKernelGGL((k_probe_mfma<0, 2>), grid, block, 0, s, iters, 1.0f, out); break;
    case 1: hipLaunchKernelGGL((k_probe_mfma<1, 2>), grid, block, 0, s, iters, 1.0f, out); break;
    case 2: hipLaunchKernelGGL((k_probe_mfma<2, 2>), grid, block, 0, s, iters, 1.0f, out); break;
    case 3: hipLaunchKernelGGL((k_probe_mfma<3, 2>), grid, block, 0, s, iters, 1.0f, out); break;
    case 4: hipLaunchKernelGGL((k_probe_mfma<2, 4>), grid, block, 0, s, iters, 1.0f, out); break;
    default: hipLaunchKernelGGL((k_probe_mfma<3, 4>), grid, block, 0, s, iters, 1.0f, out); break;
  }
  return status(hipGetLastError());
}

int hsq_probe_read(const void *src, size_t bytes, int blocks, int32_t *sink, void *stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || blocks < 1) return -1;
  if (!aligned16(src) || !aligned16(sink)) return -3;
  hipLaunchKernelGGL(k_probe_read, dim3((unsigned)blocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     (const v4u *)src, bytes / 16, sink);
  return status(hipGetLastError());
}

int hsq_probe_copy(const void *src, size_t bytes, int blocks, void *dst, void *stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0 || blocks < 1) return -1;
  if (!aligned16(src) || !aligned16(dst)) return -3;
  hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)blocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     (const v4u *)src, bytes / 16, (v4u *)dst);
  return status(hipGetLastError());
}

}  // extern "C"

// pack.hip -- K0: residual codes (K x N int8) <-> the packed blob the
// contraction kernels stream (layout version 2, described in
// hsq_internal.h): tiled nibbles, then the same codes as int8 operand bytes.
// Offline, once per weight; one thread per 16-byte lane slot.
#include "hsq_internal.h"

namespace hsq {

namespace {

// Code of input channel k, output column n (0 outside the matrix).
__device__ __forceinline__ int code_at(const int8_t *codes, int K, int N, int k, int n) {
  return (k < K && n < N) ? (int)codes[(size_t)k * N + n] : 0;
}

// One thread per 16-byte slot of the nibble part (a group pair of one lane
// slot); it also writes the slot's two 16-byte int8 operand slots (one per
// group of the pair) of the second part.
__global__ void k_pack(const int8_t *__restrict__ codes, int K, int N, int NT, int GP,
                       uint8_t *__restrict__ packed, uint8_t *__restrict__ ops, int *__restrict__ status) {
  size_t slot = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte slot
  size_t nslots = (size_t)NT * GP * 64;
  if (slot >= nslots) return;
  int lane = (int)(slot % 64);
  size_t blk = slot / 64;
  int gp = (int)(blk % GP);
  int nt = (int)(blk / GP);
  int n = nt * kTile + lane % 16;
  int bad = 0;
  uint32_t out[4];
  for (int h = 0; h < 2; ++h) {
    int kb = (2 * gp + h) * kGroup + 16 * (lane / 16);
    uint32_t o[4];
    for (int d = 0; d < 4; ++d) {          // operand bytes p = 4d .. 4d+3: 16 * code
      uint32_t w = 0;
      for (int b = 0; b < 4; ++b)
        w |= (uint32_t)(uint8_t)(16 * code_at(codes, K, N, kb + 4 * d + b, n)) << (8 * b);
      o[d] = w;
    }
    *reinterpret_cast<uint4 *>(ops + (((size_t)nt * 2 * GP + 2 * gp + h) * 64 + lane) * 16) =
        make_uint4(o[0], o[1], o[2], o[3]);
    for (int d = 0; d < 2; ++d) {          // dword d covers bytes 4d .. 4d+3
      uint32_t w = 0;
      for (int b = 0; b < 4; ++b) {
        int hi = code_at(codes, K, N, kb + 8 * d + b, n);
        int lo = code_at(codes, K, N, kb + 8 * d + 4 + b, n);
        bad |= (hi < -8) | (hi > 7) | (lo < -8) | (lo > 7);
        w |= ((uint32_t)(((hi & 0xF) << 4) | (lo & 0xF))) << (8 * b);
      }
      out[2 * h + d] = w;
    }
  }
  *reinterpret_cast<uint4 *>(packed + slot * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  if (bad) *status = 1;  // benign race: every writer stores the same value
}

__global__ void k_clear_status(int *__restrict__ status) { *status = 0; }

__global__ void k_unpack(const uint8_t *__restrict__ packed, int K, int N, int GP,
                         int8_t *__restrict__ codes) {
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // one code
  if (idx >= (size_t)K * N) return;
  int k = (int)(idx / N), n = (int)(idx % N);
  int g = k / kGroup, kk = k % kGroup;
  int lane = (n % 16) + 16 * (kk / 16);
  int p = kk % 16;
  size_t slot = ((size_t)(n / 16) * GP + g / 2) * 64 + lane;
  const uint8_t *s = packed + slot * 16 + 8 * (g % 2);
  int byte, high;
  if (p < 4)       { byte = p;     high = 1; }
  else if (p < 8)  { byte = p - 4; high = 0; }
  else if (p < 12) { byte = p - 4; high = 1; }
  else             { byte = p - 8; high = 0; }
  int nib = high ? (s[byte] >> 4) : (s[byte] & 0xF);
  codes[idx] = (int8_t)((nib ^ 8) - 8);
}

}  // namespace

hipError_t launch_pack(const int8_t *codes, int K, int N, uint8_t *packed, int *status,
                       hipStream_t s) {
  int NT = ceil_div(N, kTile), GP = padded_groups(K) / 2;
  size_t nslots = (size_t)NT * GP * 64;
  // the status word is cleared by a kernel, not a memset, so that the pack
  // call can be captured in a HIP graph as kernel nodes only
  hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(1), 0, s, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned blocks = (unsigned)((nslots + 255) / 256);
  hipLaunchKernelGGL(k_pack, dim3(blocks), dim3(256), 0, s, codes, K, N, NT, GP, packed,
                     packed + nibble_bytes(K, N), status);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int K, int N, int8_t *codes, hipStream_t s) {
  int GP = padded_groups(K) / 2;
  size_t n = (size_t)K * N;
  unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(k_unpack, dim3(blocks), dim3(256), 0, s, packed, K, N, GP, codes);
  return hipGetLastError();
}

}  // namespace hsq

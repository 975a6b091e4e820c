// Tile selection of block-sparse attention over 64-token tiles (the coarse stage
// of video sparse attention): tile means of q and k, coarse scores between the
// means, and per query tile the key tiles of highest score.
//
// The selection is an integer decided by floating point, so its arithmetic is
// fixed: means are float32 sums in token order divided by the token count,
// scores are float32 products and sums in dimension order (no fused
// multiply-add), -0 counts as +0 and NaN as the lowest score, and equal scores
// keep the lower tile index. These kernels are small next to the attention (a
// few percent of its time at sparsity 0.8) and are written for clarity.
#include "common.hpp"

namespace vdit {
namespace {

// One wave per (tile, entry * head): lane l sums dimensions [E l, E l + E).
template <int D>
__global__ void __launch_bounds__(64) vsa_mean_kernel(VsaMeanArgs a) {
  constexpr int E = D / 64;
  const int t = blockIdx.x;
  const int bh = blockIdx.y;
  const int bat = bh / a.hc;
  const int head = bh - bat * a.hc;
  const int r0 = t * 64;
  const int cnt = min(64, a.n - r0);
  const __bf16* p = a.x + bat * a.batch + (int64_t)head * D + (int64_t)r0 * a.row + threadIdx.x * E;
  float s[E];
#pragma unroll
  for (int e = 0; e < E; ++e) s[e] = 0.0f;
  for (int r = 0; r < cnt; ++r) {
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = __fadd_rn(s[e], (float)p[(int64_t)r * a.row + e]);
  }
  float* m = a.mean + ((int64_t)bh * a.tiles + t) * D + threadIdx.x * E;
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = __fdiv_rn(s[e], (float)cnt);
}

// 64 x 64 block of coarse scores per workgroup; thread (ty, tx) owns rows
// ty + 16 x and columns tx + 16 y. Every score is one running float32 sum over
// the dimensions in order.
__global__ void __launch_bounds__(256) vsa_score_kernel(VsaSelectArgs a) {
  __shared__ float qs[64][33];
  __shared__ float ks[64][33];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const float* qm = a.qm + (int64_t)bh * a.tq * a.d;
  const float* km = a.km + (int64_t)bh * a.tk * a.d;
  float acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.0f;
  for (int c0 = 0; c0 < a.d; c0 += 32) {
    for (int e = threadIdx.x; e < 64 * 32; e += 256) {
      const int r = e >> 5, c = e & 31;
      qs[r][c] = i0 + r < a.tq ? qm[(int64_t)(i0 + r) * a.d + c0 + c] : 0.0f;
      ks[r][c] = j0 + r < a.tk ? km[(int64_t)(j0 + r) * a.d + c0 + c] : 0.0f;
    }
    __syncthreads();
    for (int c = 0; c < 32; ++c) {
      float qv[4], kv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        qv[x] = qs[ty + 16 * x][c];
        kv[x] = ks[tx + 16 * x][c];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = __fadd_rn(acc[x][y], __fmul_rn(qv[x], kv[y]));
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int i = i0 + ty + 16 * x, j = j0 + tx + 16 * y;
      if (i < a.tq && j < a.tk) a.s[((int64_t)bh * a.tq + i) * a.tk + j] = acc[x][y];
    }
}

// Ascending bitonic sort of n (a power of two) 64-bit keys in LDS by the whole
// workgroup; every thread handles n / 2 / blockDim.x compare-exchanges per pass.
__device__ void bitonic_sort(uint64_t* keys, int n) {
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
        const int i = ((t & ~(j - 1)) << 1) | (t & (j - 1));  // bit j of i is clear
        const int l = i + j;
        const uint64_t x = keys[i], y = keys[l];
        if ((x > y) == ((i & k) == 0)) {
          keys[i] = y;
          keys[l] = x;
        }
      }
      __syncthreads();
    }
}

// One workgroup per (query tile, entry * head). Key of tile j: the score mapped
// to an unsigned integer of the same order, complemented (highest score first),
// in the upper 32 bits and j in the lower, so an ascending sort ranks by score
// and then by tile index. The first `keep` keys are the kept tiles; a second
// sort puts their indices in ascending order.
__global__ void __launch_bounds__(256) vsa_select_kernel(VsaSelectArgs a, int p2) {
  extern __shared__ uint64_t keys[];
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const float* row = a.s + ((int64_t)bh * a.tq + i) * a.tk;
  for (int j = threadIdx.x; j < p2; j += blockDim.x) {
    uint64_t key = ~0ull;
    if (j < a.tk) {
      float v = __fadd_rn(row[j], 0.0f);  // -0 -> +0
      if (v != v) v = -__builtin_inff();
      uint32_t u = __float_as_uint(v);
      u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      key = ((uint64_t)(~u) << 32) | (uint32_t)j;
    }
    keys[j] = key;
  }
  __syncthreads();
  bitonic_sort(keys, p2);
  int pk = 1;
  while (pk < a.keep) pk <<= 1;
  for (int p = threadIdx.x; p < pk; p += blockDim.x) keys[p] = p < a.keep ? (keys[p] & 0xffffffffull) : ~0ull;
  __syncthreads();
  bitonic_sort(keys, pk);
  int32_t* o = a.tiles + ((int64_t)bh * a.tq + i) * a.keep;
  for (int p = threadIdx.x; p < a.keep; p += blockDim.x) o[p] = (int32_t)keys[p];
}

}  // namespace

hipError_t launch_vsa_means(const VsaMeanArgs& a, int head_dim, hipStream_t s) {
  if (a.tiles <= 0 || a.bh <= 0 || a.bh > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.tiles, (unsigned)a.bh);
  if (head_dim == 128)
    hipLaunchKernelGGL(vsa_mean_kernel<128>, grid, dim3(64), 0, s, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(vsa_mean_kernel<64>, grid, dim3(64), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_vsa_select(const VsaSelectArgs& a, hipStream_t s) {
  if (a.tq <= 0 || a.tk <= 0 || a.tk > kVsaMaxTiles || a.keep < 1 || a.keep > a.tk || a.bh <= 0 ||
      a.bh > 65535 || a.d % 32 != 0 || a.tq > 0x7fffffff)
    return hipErrorInvalidValue;
  const dim3 sgrid((unsigned)((a.tk + 63) / 64), (unsigned)((a.tq + 63) / 64), (unsigned)a.bh);
  hipLaunchKernelGGL(vsa_score_kernel, sgrid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int p2 = 2;
  while (p2 < a.tk) p2 <<= 1;
  hipLaunchKernelGGL(vsa_select_kernel, dim3((unsigned)a.tq, (unsigned)a.bh), dim3(256), (size_t)p2 * 8, s, a, p2);
  return hipGetLastError();
}

}  // namespace vdit

// Tile selection of block-sparse attention over 64-token tiles (the coarse stage
// of video sparse attention): tile means of q and k, coarse scores between the
// means, and per query tile the key tiles of highest score. A tile is a run of 64
// consecutive tokens, or a 4 x 4 x 4 cube of the latent grid (CubeGeom).
//
// The selection is an integer decided by floating point, so its arithmetic is
// fixed: means are float32 sums in token order divided by the token count,
// scores are float32 products and sums in dimension order (no fused
// multiply-add), -0 counts as +0 and NaN as the lowest score, and equal scores
// keep the lower tile index. These kernels are small next to the attention (a
// few percent of its time at sparsity 0.8).
#include "common.hpp"

namespace vdit {
namespace {

// One wave per (tile, entry * head): lane l sums dimensions [E l, E l + E) over the
// tile's tokens in ascending order.
template <int D>
__global__ void __launch_bounds__(64) vsa_mean_kernel(VsaMeanArgs a) {
  constexpr int E = D / 64;
  const int t = blockIdx.x;
  const int bh = blockIdx.y;
  const int bat = bh / a.hc;
  const int head = bh - bat * a.hc;
  float s[E];
#pragma unroll
  for (int e = 0; e < E; ++e) s[e] = 0.0f;
  int cnt;
  if (a.cube.on) {
    // cube t: its tokens in ascending order, 16 loads in flight, the sums in order
    const Cube cb = cube_at(a.cube, t);
    cnt = cb.len;
    const __bf16* base = a.x + bat * a.batch + (int64_t)head * D + threadIdx.x * E;
    for (int r0 = 0; r0 < cnt; r0 += 16) {
      __bf16 x[16][E];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = r0 + r < cnt ? cube_token(a.cube, cb, r0 + r) : 0;
#pragma unroll
        for (int e = 0; e < E; ++e) x[r][e] = base[(int64_t)tok * a.row + e];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r0 + r < cnt)
#pragma unroll
          for (int e = 0; e < E; ++e) s[e] = __fadd_rn(s[e], (float)x[r][e]);
    }
    float* m = a.mean + ((int64_t)bh * a.tiles + t) * D + threadIdx.x * E;
#pragma unroll
    for (int e = 0; e < E; ++e) m[e] = __fdiv_rn(s[e], (float)cnt);
    return;
  }
  const int r0 = t * 64;
  cnt = min(64, a.n - r0);
  const __bf16* p = a.x + bat * a.batch + (int64_t)head * D + (int64_t)r0 * a.row + threadIdx.x * E;
  if (cnt == 64) {
    // full tile: all 64 loads in flight in groups of 16, the sums still in token order
#pragma unroll
    for (int r0 = 0; r0 < 64; r0 += 16) {
      __bf16 x[16][E];
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) x[r][e] = p[(int64_t)(r0 + r) * a.row + e];
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = __fadd_rn(s[e], (float)x[r][e]);
    }
  } else {
    for (int r = 0; r < cnt; ++r) {
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] = __fadd_rn(s[e], (float)p[(int64_t)r * a.row + e]);
    }
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

// Block-wide inclusive prefix sum of one value per thread (256 threads).
__device__ uint32_t block_scan(uint32_t v, uint32_t* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == 63) wtot[w] = v;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) add += k < w ? wtot[k] : 0u;
  __syncthreads();
  return v + add;
}

// Exclusive rank of a true flag among the true flags of lower threads, and the
// block's total (256 threads).
__device__ uint32_t flag_rank(bool f, uint32_t* wtot, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(f);
  const uint32_t below = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wtot[w] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t x = wtot[k];
    off += k < w ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return off + below;
}

constexpr int kSelThreads = 256;
constexpr int kSelPerThread = kVsaMaxTiles / kSelThreads;

// One workgroup per (query tile, entry * head). Thread t holds the keys of
// tiles t, t + 256, ...: the score mapped to an unsigned integer whose order is
// the reverse of the score order, so the kept tiles are the `keep` smallest keys
// (equal keys: lower tile first). A radix select over the four 8-bit digits,
// most significant first (a histogram of the keys that match the digits found
// so far, then the bin holding the wanted rank), gives the value of the
// keep-th smallest key and how many keys equal to it are kept; a pass in tile
// order then writes the kept tiles ascending.
__global__ void __launch_bounds__(kSelThreads) vsa_select_kernel(VsaSelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wtot[4];
  __shared__ uint32_t found[2];
  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const float* row = a.s + ((int64_t)bh * a.tq + i) * a.tk;
  const int per = (a.tk + kSelThreads - 1) / kSelThreads;
  uint32_t key[kSelPerThread];
#pragma unroll
  for (int c = 0; c < kSelPerThread; ++c) {
    const int j = c * kSelThreads + tid;
    uint32_t kv = 0xffffffffu;  // above every score's key
    if (j < a.tk) {
      float v = __fadd_rn(row[j], 0.0f);  // -0 -> +0
      if (v != v) v = -__builtin_inff();
      uint32_t u = __float_as_uint(v);
      u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending with the score
      kv = ~u;
    }
    key[c] = kv;
  }
  uint32_t prefix = 0, r = (uint32_t)a.keep;  // r: rank still wanted among keys matching prefix
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int sh = 24 - 8 * p;
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kSelPerThread; ++c) {
      const uint32_t k = key[c];
      const bool match = c * kSelThreads + tid < a.tk && (p == 0 || ((k ^ prefix) >> (sh + 8)) == 0);
      if (match) atomicAdd(&hist[(k >> sh) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t cnt = hist[tid];
    const uint32_t incl = block_scan(cnt, wtot);
    if (incl - cnt < r && r <= incl) {
      found[0] = (uint32_t)tid;
      found[1] = r - (incl - cnt);
    }
    __syncthreads();
    prefix |= found[0] << sh;
    r = found[1];
    __syncthreads();
  }
  int32_t* o = a.tiles + ((int64_t)bh * a.tq + i) * a.keep;
  uint32_t base_eq = 0, base_out = 0;
#pragma unroll
  for (int c = 0; c < kSelPerThread; ++c) {
    if (c < per) {  // the same for every thread: the barriers inside stay uniform
      const int j = c * kSelThreads + tid;
      const bool valid = j < a.tk;
      const bool eq = valid && key[c] == prefix;
      uint32_t n_eq, n_kept;
      const uint32_t rank_eq = base_eq + flag_rank(eq, wtot, n_eq);
      const bool kept = valid && (key[c] < prefix || (eq && rank_eq < r));
      const uint32_t pos = base_out + flag_rank(kept, wtot, n_kept);
      if (kept) o[pos] = j;
      base_eq += n_eq;
      base_out += n_kept;
    }
  }
}

}  // namespace

hipError_t launch_vsa_means(const VsaMeanArgs& a, int head_dim, hipStream_t s) {
  if (a.tiles <= 0 || a.bh <= 0 || a.bh > 65535) return hipErrorInvalidValue;
  if (a.cube.on && (a.tiles != a.cube.n || (int64_t)a.cube.t * a.cube.h * a.cube.w != a.n)) return hipErrorInvalidValue;
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
  hipLaunchKernelGGL(vsa_select_kernel, dim3((unsigned)a.tq, (unsigned)a.bh), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace vdit

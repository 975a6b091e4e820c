// Bandwidth-bound kernels around the attention kernel:
//   * v range: partial maxima of |v| over the valid keys of each (entry, head);
//   * prepare: v of the head share, scaled by the power of two 2^e that brings its
//     maximum into [2^14, 2^15), -> float16 V^T tiles in the workspace (keys
//     permuted inside groups of 16 to match the weight layout of the attention
//     kernel, zero past the valid keys), and with RoPE the rotated keys;
//   * quantize (int8 q.k): symmetric int8 codes and float32 scales of q (128
//     tokens per block, softmax scale folded in) and k (64 keys per block);
//   * pack / unpack: [n, Ht, d] <-> [G, n, Ht/G, d] for the Ulysses exchange;
//   * rope probe: the (t, y, x, band, i) index map as the kernels compute it.
#include "common.hpp"

namespace vdit {
namespace {

// Position of key k (0..63) inside a prepared 64-key V^T tile: bits 2 and 3 of
// the index are swapped. In the 32x32 accumulator of S^T a lane of half h holds,
// for 16 consecutive keys, keys {4h..4h+3} then {8+4h..8+4h+3}; after the swap
// those eight keys are adjacent, so one 16-byte read gives the lane its operand.
__device__ __forceinline__ int vt_position(int k) {
  return (k & ~15) | (k & 3) | ((k >> 1) & 4) | ((k << 1) & 8);
}

// Partial maximum of |v| over part blockIdx.x of the valid keys of (entry, head)
// blockIdx.y; each part is a contiguous run of keys (possibly empty: then 0).
template <int D>
__global__ void __launch_bounds__(256) vrange_kernel(PrepArgs a) {
  constexpr int kChunks = D / 8;
  __shared__ float red[4];
  const int part = blockIdx.x;
  const int bh = blockIdx.y;
  const int bat = bh / a.hc;
  const int head = bh - bat * a.hc;
  const int kv_len = a.kv_len[bat];
  const int per = (kv_len + kVParts - 1) / kVParts;
  const int k0 = part * per;
  const int k1 = min(kv_len, k0 + per);
  const __bf16* vsrc = a.v + bat * a.kv_batch + (int64_t)head * a.kv_head;
  float m = 0.0f;
  const int total = max(k1 - k0, 0) * kChunks;
  // four independent 16-byte loads per thread in flight
  for (int c0 = threadIdx.x; c0 < total; c0 += 4 * 256) {
    bf16x8 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * 256;
      v[u] = c < total ? *reinterpret_cast<const bf16x8*>(vsrc + (int64_t)(k0 + c / kChunks) * a.kv_row + (c % kChunks) * 8)
                       : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[u][e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) a.vpart[(int64_t)bh * kVParts + part] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One 64-key tile of (entry, head) bh: v scaled by 2^vsh -> float16 V^T tile, and
// the tile's k in cube order (cube tiles) or rotated (RoPE). Uses `tr` in LDS and
// one barrier; the caller separates consecutive calls with another.
template <int D, bool ROPE>
__device__ __forceinline__ void prepare_tile(const PrepArgs& a, int tile, int bh, int vsh, _Float16* tr) {
  constexpr int kChunks = D / 8;
  constexpr int kLoads = kBlockN * kChunks / 256;
  constexpr int kPad = kBlockN + 8;
  const int bat = bh / a.hc;
  const int head = bh - bat * a.hc;
  const int tid = threadIdx.x;
  const int kv_len = a.kv_len[bat];
  // latent-grid cubes: this tile holds cube `tile`, slot kl its kl-th token
  Cube cb{};
  if (a.cube.on) cb = cube_at(a.cube, tile);
  auto key_of = [&](int kl) -> int {
    if (a.cube.on) return kl < cb.len ? cube_token(a.cube, cb, kl) : -1;
    const int key = tile * kBlockN + kl;
    return key < kv_len ? key : -1;
  };
  const __bf16* vsrc = a.v + bat * a.kv_batch + (int64_t)head * a.kv_head;

  // thread: kLoads consecutive keys (one 16-byte chunk of each), so that each of
  // its dimensions goes to LDS as one write of kLoads float16 (consecutive keys stay
  // adjacent under vt_position) instead of kLoads 2-byte writes
  {
    static_assert(kLoads == 2 || kLoads == 4, "keys per thread");
    typedef _Float16 f16xg __attribute__((ext_vector_type(kLoads)));
    const int kg = tid / kChunks;
    const int ch = tid % kChunks;
    bf16x8 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int key = key_of(kg * kLoads + j);
      v[j] = key >= 0 ? *reinterpret_cast<const bf16x8*>(vsrc + (int64_t)key * a.kv_row + ch * 8) : bf16x8{};
    }
    const int pos = vt_position(kg * kLoads);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f16xg w;
#pragma unroll
      for (int j = 0; j < kLoads; ++j) w[j] = (_Float16)__builtin_amdgcn_ldexpf((float)v[j][e], vsh);
      *reinterpret_cast<f16xg*>(&tr[(ch * 8 + e) * kPad + pos]) = w;
    }
  }
  __syncthreads();
  _Float16* dst = a.vt + (int64_t)bh * a.vt_head + (int64_t)tile * (D * kBlockN);
#pragma unroll
  for (int i = 0; i < D * (kBlockN / 8) / 256; ++i) {
    const int qd = i * 256 + tid;
    const int row = qd >> 3;
    const int ch = qd & 7;
    *reinterpret_cast<u32x4*>(dst + row * kBlockN + ch * 8) =
        *reinterpret_cast<const u32x4*>(&tr[row * kPad + ch * 8]);
  }

  if (!ROPE && a.cube.on) {
    // k in cube order: slot kl of tile `tile` holds the cube's kl-th key (zero past
    // its token count; the attention kernel masks those scores)
    const __bf16* ksrc = a.k + bat * a.kv_batch + (int64_t)head * a.kv_head;
    __bf16* kdst = a.kr + (int64_t)bh * a.kr_head + (int64_t)tile * kBlockN * D;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int qd = i * 256 + tid;
      const int kl = qd / kChunks;
      const int ch = qd % kChunks;
      const int key = key_of(kl);
      bf16x8 v = bf16x8{};
      if (key >= 0) v = *reinterpret_cast<const bf16x8*>(ksrc + (int64_t)key * a.kv_row + ch * 8);
      *reinterpret_cast<bf16x8*>(kdst + kl * D + ch * 8) = v;
    }
  }

  if constexpr (ROPE) {
    const __bf16* ksrc = a.k + bat * a.kv_batch + (int64_t)head * a.kv_head;
    __bf16* kdst = a.kr + (int64_t)bh * a.kr_head;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int qd = i * 256 + tid;
      const int kl = qd / kChunks;
      const int ch = qd % kChunks;
      const int key = tile * kBlockN + kl;
      bf16x8 v = bf16x8{};
      if (key < kv_len) {
        v = *reinterpret_cast<const bf16x8*>(ksrc + (int64_t)key * a.kv_row + ch * 8);
        int t, y, x;
        rope_token_pos(a.rope, key, t, y, x);
        v = rope_chunk(a.rope, v, ch * 8, t, y, x);
      }
      *reinterpret_cast<bf16x8*>(kdst + (int64_t)key * D + ch * 8) = v;
    }
  }
}

template <int D, bool ROPE>
__global__ void __launch_bounds__(256) prepare_kernel(PrepArgs a) {
  constexpr int kPad = kBlockN + 8;  // float16 per LDS row: 144 bytes, keeps 16-byte alignment
  __shared__ __attribute__((aligned(16))) _Float16 tr[D * kPad];

  const int tile = blockIdx.x;
  const int bh = blockIdx.y;               // batch entry * hc + local head
  const int bat = bh / a.hc;
  const int tid = threadIdx.x;
  // tiles past this entry's keys are never read by the attention kernel
  if (!a.cube.on && tile * kBlockN >= a.kv_len[bat]) return;
  // the scaling of this (entry, head): every wave combines the partial maxima
  static_assert(kVParts == kWave, "one partial maximum per lane");
  float amax = a.vpart[(int64_t)bh * kVParts + (tid & 63)];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const int vsh = v_scale_exp(amax);
  if (tile == 0 && tid == 0) {
    a.vexp[bh] = vsh;
    if (a.retry_cnt) {
      a.retry_cnt[2 * bh] = 0;
      a.retry_cnt[2 * bh + 1] = 0;
    }
  }
  prepare_tile<D, ROPE>(a, tile, bh, vsh, tr);
}

// Short key sequences (at most kSmallKeys keys per entry, not cube-tiled): one
// workgroup per (entry, head) finds max |v| over the valid keys and then prepares
// every key tile, one launch instead of the range and prepare launches; the values
// written are the same.
template <int D, bool ROPE>
__global__ void __launch_bounds__(256) prepare_short_kernel(PrepArgs a) {
  constexpr int kChunks = D / 8;
  constexpr int kPad = kBlockN + 8;
  __shared__ __attribute__((aligned(16))) _Float16 tr[D * kPad];
  __shared__ float red[4];
  const int bh = blockIdx.x;
  const int bat = bh / a.hc;
  const int head = bh - bat * a.hc;
  const int tid = threadIdx.x;
  const int kv_len = a.kv_len[bat];
  const __bf16* vsrc = a.v + bat * a.kv_batch + (int64_t)head * a.kv_head;
  float m = 0.0f;
  const int total = kv_len * kChunks;
  for (int c0 = tid; c0 < total; c0 += 4 * 256) {
    bf16x8 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * 256;
      v[u] = c < total ? *reinterpret_cast<const bf16x8*>(vsrc + (int64_t)(c / kChunks) * a.kv_row + (c % kChunks) * 8)
                       : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[u][e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int vsh = v_scale_exp(amax);
  if (tid == 0) {
    a.vexp[bh] = vsh;
    if (a.retry_cnt) {
      a.retry_cnt[2 * bh] = 0;
      a.retry_cnt[2 * bh + 1] = 0;
    }
  }
  const int ntiles = (kv_len + kBlockN - 1) / kBlockN;
  for (int tile = 0; tile < ntiles; ++tile) {
    prepare_tile<D, ROPE>(a, tile, bh, vsh, tr);
    __syncthreads();  // the next tile rewrites tr
  }
}

// Symmetric int8 codes of one block of consecutive tokens of one (entry, head):
// blockIdx.z = 0 quantizes q, multiplied by the softmax scale, in blocks of 128
// tokens; blockIdx.z = 1 quantizes k in blocks of 64 valid keys. Each decision is
// float32, in this order: x = float(bf16) (* softmax scale for q); amax = max |x|
// over the block; scale = amax / 127 (IEEE division), replaced by 1 below 2^-100;
// code = rint(x / scale) (IEEE division, ties to even), clamped to [-127, 127].
template <int D>
__global__ void __launch_bounds__(256) quantize_kernel(QuantArgs a) {
  constexpr int kChunks = D / 8;                   // 8-element chunks per token
  constexpr int kPer = kQuantQ * kChunks / 256;    // chunks per thread, q blocks
  __shared__ float red[4];
  const bool is_q = blockIdx.z == 0;
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int bat = bh / a.hc;
  const int head = bh - bat * a.hc;
  const int n = is_q ? a.nq : a.kv_len[bat];
  const int per_block = is_q ? kQuantQ : kQuantK;
  if (blk * per_block >= n) return;                // whole workgroup
  const int r0 = blk * per_block;
  const int total = min(per_block, n - r0) * kChunks;
  const __bf16* src = is_q ? a.q + bat * a.q_batch + (int64_t)head * a.head
                           : a.k + bat * a.k_batch + (int64_t)head * a.head;
  const int64_t row = is_q ? a.q_row : a.k_row;
  const int tid = threadIdx.x;

  float x[kPer][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = i * 256 + tid;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] = 0.0f;
    if (c < total) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + (int64_t)(r0 + c / kChunks) * row + (c % kChunks) * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[i][e] = is_q ? (float)v[e] * a.sm_scale : (float)v[e];
        amax = fmaxf(amax, fabsf(x[i][e]));
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float scale = __fdiv_rn(amax, 127.0f);
  if (!(scale >= 0x1p-100f)) scale = 1.0f;
  if (tid == 0) (is_q ? a.qsc + (int64_t)bh * a.nq_blocks : a.ksc + (int64_t)bh * a.nk_blocks)[blk] = scale;

  int8_t* dst = (is_q ? a.qc + bh * a.qc_bh : a.kc + bh * a.kc_bh) + (int64_t)r0 * D;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = i * 256 + tid;
    if (c < total) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = fminf(fmaxf(__builtin_rintf(__fdiv_rn(x[i][e], scale)), -127.0f), 127.0f);
        w[e >> 2] |= (uint32_t)(uint8_t)(int8_t)(int)qv << (8 * (e & 3));
      }
      *reinterpret_cast<uint2*>(dst + (int64_t)c * 8) = make_uint2(w[0], w[1]);
    }
  }
}

// One workgroup per token row: moves that token's Ht * d elements between the
// [n, Ht, d] and [G, n, Ht/G, d] layouts in 16-byte chunks.
__global__ void __launch_bounds__(256) pack_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n, int32_t ht, int32_t cpr, int32_t hg, int32_t unpack) {
  const int64_t t = blockIdx.x;
  const int32_t row_chunks = ht * cpr;   // chunks of one token
  const int32_t grp_chunks = hg * cpr;   // chunks of one token inside one group
  for (int32_t i = threadIdx.x; i < row_chunks; i += 256) {
    const int32_t g = i / grp_chunks;
    const int32_t r = i - g * grp_chunks;
    const int64_t flat = t * row_chunks + i;                  // [n, Ht, d] index
    const int64_t grouped = (g * n + t) * grp_chunks + r;     // [G, n, Ht/G, d] index
    // streamed once: non-temporal loads and stores keep the copy out of the caches
    // (~10% more bandwidth than cached accesses at these sizes)
    if (unpack)
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + grouped), dst + flat);
    else
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + flat), dst + grouped);
  }
}

__global__ void __launch_bounds__(256) rope_probe_kernel(RopeGeom g, int32_t nq, int32_t pairs, int32_t* out) {
  const int64_t total = (int64_t)nq * pairs;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int32_t n = (int32_t)(idx / pairs);
    const int32_t p = (int32_t)(idx - (int64_t)n * pairs);
    int t, y, x;
    rope_token_pos(g, n, t, y, x);
    const RopeIndex r = rope_pair_index(g, p, t, y, x);
    int32_t* o = out + idx * 5;
    o[0] = t; o[1] = y; o[2] = x; o[3] = r.band; o[4] = r.i;
  }
}

template <int D, bool ROPE>
hipError_t launch_prepare_t(const PrepArgs& a, hipStream_t s) {
  if (!a.cube.on && a.n_ktiles * kBlockN <= kSmallKeys) {
    hipLaunchKernelGGL((prepare_short_kernel<D, ROPE>), dim3(a.hc * a.batch), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((vrange_kernel<D>), dim3(kVParts, a.hc * a.batch), dim3(256), 0, s, a);
  hipLaunchKernelGGL((prepare_kernel<D, ROPE>), dim3(a.n_ktiles, a.hc * a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare(const PrepArgs& a, int head_dim, bool rope_k, hipStream_t s) {
  if (a.n_ktiles <= 0 || a.hc <= 0 || a.batch <= 0 || a.batch > kMaxBatch || (int64_t)a.hc * a.batch > 65535 ||
      !a.vpart || !a.vexp)
    return hipErrorInvalidValue;
  if (a.cube.on && (rope_k || !a.kr || a.n_ktiles != a.cube.n)) return hipErrorInvalidValue;
  if (head_dim == 128) return rope_k ? launch_prepare_t<128, true>(a, s) : launch_prepare_t<128, false>(a, s);
  if (head_dim == 64) return rope_k ? launch_prepare_t<64, true>(a, s) : launch_prepare_t<64, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_quantize(const QuantArgs& a, int head_dim, hipStream_t s) {
  if (head_dim != 128 || a.hc <= 0 || a.batch <= 0 || a.batch > kMaxBatch || (int64_t)a.hc * a.batch > 65535)
    return hipErrorInvalidValue;
  const int nblk = a.nq_blocks > a.nk_blocks ? a.nq_blocks : a.nk_blocks;
  hipLaunchKernelGGL(quantize_kernel<128>, dim3(nblk, a.hc * a.batch, 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, void* dst, int64_t n, int32_t ht, int32_t d, int32_t groups,
                       bool unpack, hipStream_t s) {
  if (n <= 0 || n > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)n), dim3(256), 0, s, reinterpret_cast<const u32x4*>(src),
                     reinterpret_cast<u32x4*>(dst), n, ht, d / 8, ht / groups, unpack ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_rope_probe(const RopeGeom& g, int32_t nq, int32_t head_dim, int32_t* out, hipStream_t s) {
  const int64_t total = (int64_t)nq * (head_dim / 2);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(rope_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g, nq, head_dim / 2, out);
  return hipGetLastError();
}

}  // namespace vdit

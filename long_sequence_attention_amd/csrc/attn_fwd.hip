// Flash-style attention forward for gfx950 (CDNA4), bf16 q/k, fp16 weights and v.
//
// Work split: one workgroup = WAVES waves = BLOCK_M = WAVES * QB * 32 queries of one head;
// it streams all valid keys of that head in tiles of 64 keys through a double-
// buffered LDS stage (K tile row-major, V^T tile prepared in the workspace).
//
// Per wave and key tile the scores are formed transposed, S^T = K * Q^T, with
// v_mfma_f32_32x32x16_bf16: the A operand is a 32-key x 16-dim slice of K read
// from LDS, the B operand is the wave's queries held in registers for the whole
// loop. In the 32x32 accumulator layout lane l holds query (l % 32) and 16 of
// its keys, the other 16 in lane l ^ 32, so the per-query maximum and sum need
// one cross-half exchange only. The float16 weights P^T stay in the same lanes
// and serve directly as the B operand of O^T += V^T * P^T
// (v_mfma_f32_32x32x16_f16); the workspace stores V^T with the key order inside
// each group of 16 permuted (bits 2 and 3 of the key index swapped) so that the
// A operand for a lane is one 16-byte LDS read.
//
// Softmax runs in the log2 domain (c = scale * log2 e) with a running maximum
// that is only raised when a tile's maximum exceeds it by more than 2^8, so the
// rescale of O is rare after the first tiles; the row sum is taken from the
// rounded float16 weights (v_dot2), the same values the product uses.
#include "common.hpp"

namespace vdit {
namespace {

template <int D, int QB, int WAVES>
struct FwdCfg {
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kBlockM = kWaves * QB * 32;
  static constexpr int kKChunks = D / 8;                          // 16-byte chunks per K row
  static constexpr int kKTile = kBlockN * D * 2;                   // bytes
  static constexpr int kVTile = D * kBlockN * 2;                   // bytes
  static constexpr int kStage = kKTile + kVTile;
  static constexpr int kLds = 2 * kStage;
  static constexpr int kKLoads = kBlockN * kKChunks / kThreads;    // 16-byte loads per thread
  static constexpr int kVLoads = D * (kBlockN / 8) / kThreads;
  static constexpr int kDK = D / 16;                               // MFMA k-steps over d
  static constexpr int kDB = D / 32;                               // 32-row blocks of d
  static_assert(kKLoads >= 1 && kVLoads >= 1, "tile too small for the workgroup");
};

template <int D, int QB, int WAVES, bool ROPE>
__global__ void __launch_bounds__(WAVES * 64) attn_fwd_kernel(AttnArgs a) {
  using C = FwdCfg<D, QB, WAVES>;
  __shared__ __attribute__((aligned(16))) char lds[C::kLds];

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so that
  // each XCD walks a contiguous range of (head, query tile) and its L2 serves the
  // K/V tiles of one head to all its CUs.
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  const int per = nwg >> 3;
  const int rem = nwg & 7;
  const int id = xcd * per + (xcd < rem ? xcd : rem) + (wg >> 3);
  const int head = id / a.n_qtiles;
  const int qtile = id - head * a.n_qtiles;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- prologue: this wave's queries into registers (B operand layout), RoPE fused
  const int q0 = qtile * C::kBlockM + wave * QB * 32;
  bf16x8 qf[QB][C::kDK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = q0 + qb * 32 + l32;
    if (qi < a.nq) {
      const __bf16* qp = a.q + (int64_t)qi * a.q_row + (int64_t)head * a.q_head + 8 * hl;
      int t = 0, y = 0, x = 0;
      if constexpr (ROPE) rope_token_pos(a.rope, qi, t, y, x);
#pragma unroll
      for (int kk = 0; kk < C::kDK; ++kk) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
        if constexpr (ROPE) v = rope_chunk(a.rope, v, 16 * kk + 8 * hl, t, y, x);
        qf[qb][kk] = v;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < C::kDK; ++kk) qf[qb][kk] = bf16x8{};
    }
  }

  __shared__ int wg_retry;
  if (tid == 0) wg_retry = 0;

  const __bf16* kbase = a.k + (int64_t)head * a.k_head;
  const _Float16* vbase = a.vt + (int64_t)head * a.vt_head;
  const int kv_len = a.kv_len;
  const int ntiles = (kv_len + kBlockN - 1) / kBlockN;
  const float c = a.c;

  u32x4 kreg[C::kKLoads], vreg[C::kVLoads];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::kKLoads; ++i) {
      const int qd = i * C::kThreads + tid;
      const int row = qd / C::kKChunks;
      const int ch = qd % C::kKChunks;
      // keys past kv_len read the last valid row instead (their scores are masked),
      // so no row at or beyond kv_len is ever read
      const int key = min(t * kBlockN + row, kv_len - 1);
      kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * a.k_row + ch * 8);
    }
    const _Float16* vt = vbase + (int64_t)t * (D * kBlockN);
#pragma unroll
    for (int i = 0; i < C::kVLoads; ++i) {
      const int qd = i * C::kThreads + tid;
      vreg[i] = *reinterpret_cast<const u32x4*>(vt + qd * 8);
    }
  };
  auto lstore = [&](int stage) {
    char* kl = lds + stage * C::kStage;
    char* vl = kl + C::kKTile;
#pragma unroll
    for (int i = 0; i < C::kKLoads; ++i) {
      const int qd = i * C::kThreads + tid;
      const int row = qd / C::kKChunks;
      const int ch = qd % C::kKChunks;
      *reinterpret_cast<u32x4*>(kl + row * (D * 2) + ((ch ^ (row & (C::kKChunks - 1))) << 4)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::kVLoads; ++i) {
      const int qd = i * C::kThreads + tid;
      const int row = qd >> 3;
      const int ch = qd & 7;
      *reinterpret_cast<u32x4*>(vl + row * (kBlockN * 2) + ((ch ^ ((row >> 1) & 7)) << 4)) = vreg[i];
    }
  };

  // per-lane LDS read offsets (the XOR swizzle only depends on the lane)
  const int kswz = l32 & (C::kKChunks - 1);
  const int vswz = (l32 >> 1) & 7;
  const int krow_off = l32 * (D * 2);
  const int vrow_off = l32 * (kBlockN * 2);

  // S^T = K * Q^T for the tile in LDS stage `st`, keys past kv_len set to -inf
  auto scores = [&](int st, int t, f32x16 (&s)[QB][2]) {
    const char* kl = lds + st * C::kStage;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { s[qb][0] = f32x16{}; s[qb][1] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < C::kDK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
            kl + kb * 32 * (D * 2) + krow_off + (((2 * kk + hl) ^ kswz) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][kk], s[qb][kb], 0, 0, 0);
      }
    }
    if (t == ntiles - 1 && (kv_len & (kBlockN - 1))) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t * kBlockN + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (key >= kv_len) s[qb][kb][r] = -__builtin_inff();
          }
    }
  };
  // maximum of the scores of each query in the tile (both lane halves), times c
  auto tile_max = [&](const f32x16 (&s)[QB][2], float (&m)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][1][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m[qb] = mx * c;
    }
  };

  // One pass over all key tiles with a fixed reference m (log2 domain): weights
  // p = 2^(s*c - m) rounded to float16, O^T += V^T * P^T, l += sum of the rounded
  // weights. Entry: tile 0 is in LDS stage 0. A weight above the float16 range
  // becomes inf and makes l non-finite, which the caller checks.
  f32x16 o[QB][C::kDB];
  float l_run[QB];
  auto main_pass = [&](const float (&mref)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      l_run[qb] = 0.0f;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) o[qb][db] = f32x16{};
    }
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    for (int t = 0; t < ntiles; ++t) {
      const int st = t & 1;
      const bool more = t + 1 < ntiles;
      if (more) gload(t + 1);
      f32x16 s[QB][2];
      scores(st, t, s);
      f16x8 pf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float nm = -mref[qb];
        float lsum = 0.0f;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int kb = s4 >> 1;
          const int base = (s4 & 1) * 8;
          f16x8 pk;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            f16x2 h2;
            h2[0] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][base + e], c, nm));
            h2[1] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][base + e + 1], c, nm));
            lsum = __builtin_amdgcn_fdot2(h2, ones, lsum, false);
            pk[e] = h2[0];
            pk[e + 1] = h2[1];
          }
          pf[qb][s4] = pk;
        }
        l_run[qb] += lsum;
      }
      const char* vl = lds + st * C::kStage + C::kKTile;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
        for (int db = 0; db < C::kDB; ++db) {
          const f16x8 va = *reinterpret_cast<const f16x8*>(
              vl + db * 32 * (kBlockN * 2) + vrow_off + (((2 * s4 + hl) ^ vswz) << 4));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[qb][s4], o[qb][db], 0, 0, 0);
        }
      }
      if (more) lstore(st ^ 1);
      __syncthreads();
    }
  };

  // ---- reference maximum from the first key tile
  gload(0);
  lstore(0);
  __syncthreads();
  float mref[QB];
  {
    f32x16 s[QB][2];
    scores(0, 0, s);
    tile_max(s, mref);
  }
  main_pass(mref);

  // ---- rare path: some weight left the float16 range (a later key scored far
  // above the first tile's maximum) or the inputs were not finite. The whole
  // workgroup recomputes with the exact row maximum, so no weight exceeds 1.
  bool bad = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) bad |= !__builtin_isfinite(l_run[qb]);
  if (__any(bad) && lane == 0) wg_retry = 1;
  __syncthreads();
  if (wg_retry) {
    float mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = -__builtin_inff();
    for (int t = 0; t < ntiles; ++t) {
      gload(t);
      lstore(0);
      __syncthreads();
      f32x16 s[QB][2];
      scores(0, t, s);
      float m[QB];
      tile_max(s, m);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = fmaxf(mx[qb], m[qb]);
      __syncthreads();
    }
    gload(0);
    lstore(0);
    __syncthreads();
    main_pass(mx);
  }

  // ---- epilogue: normalise, round to bf16, store [nq, hc, d]
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = 1.0f / lt;
    const int qi = q0 + qb * 32 + l32;
    if (qi < a.nq) {
      __bf16* op = a.out + ((int64_t)qi * a.hc + head) * D + 4 * hl;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[qb][db][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(op + db * 32 + 8 * g) = w;
        }
    }
  }
}

template <int D, int QB, int WAVES, bool ROPE>
hipError_t launch_fwd_t(AttnArgs a, hipStream_t s) {
  using C = FwdCfg<D, QB, WAVES>;
  a.n_qtiles = (a.nq + C::kBlockM - 1) / C::kBlockM;
  const int64_t nwg = (int64_t)a.n_qtiles * a.hc;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_kernel<D, QB, WAVES, ROPE>), dim3((unsigned)nwg), dim3(C::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, int head_dim, bool rope_q, hipStream_t s) {
  if (head_dim == 128) return rope_q ? launch_fwd_t<128, 1, 8, true>(a, s) : launch_fwd_t<128, 1, 8, false>(a, s);
  if (head_dim == 64) return rope_q ? launch_fwd_t<64, 1, 8, true>(a, s) : launch_fwd_t<64, 1, 8, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace vdit

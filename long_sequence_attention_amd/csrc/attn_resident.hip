// Attention forward with the keys and values resident in LDS, for short key
// sequences such as the text of a cross-attention layer (every key length of the
// call at most 256 keys at d = 128, 512 at d = 64).
//
// K and V^T of one (entry, head) take 128 KB of LDS, so a workgroup stages them
// once and then streams query tiles against them: there are no per-tile direct
// loads and no barriers in the loop, and each wave runs on its own. The grid is
// persistent (at most one workgroup per CU): workgroup i takes a contiguous range
// of 256-query tiles in (entry, head, tile) order and restages K/V^T only when the
// range crosses into the next head. A wave loads the q of its next tile into the
// q registers as soon as its last score product has read them, so the load runs
// under the remaining weights, products and the epilogue.
//
// Per wave and query row the arithmetic is that of the streaming kernel (same
// products in the same order, the same fixed-reference softmax, row sums and
// rounding), so both give bit-identical rows; only the exact-maximum retry is
// decided per wave here instead of per workgroup.
#include "common.hpp"
#include "lds.hpp"

namespace vdit {
namespace {

constexpr int kResWaves = 8;
constexpr int kResThreads = kResWaves * kWave;
constexpr int kResQ = kResWaves * 32;      // queries per query tile
constexpr int kResKVBytes = 128 * 1024;    // LDS for the resident K and V^T tiles
constexpr int kResEpiBytes = 4096;         // LDS per wave for the output rows

template <int D>
struct ResCfg {
  static constexpr int kKRow = D * 2;                   // bytes per K row in LDS
  static constexpr int kKChunks = kKRow / 16;           // 16-byte chunks per K row
  static constexpr int kVRow = kBlockN * 2;             // bytes per V^T row in LDS
  static constexpr int kKTile = kBlockN * kKRow;
  static constexpr int kVTile = D * kVRow;
  static constexpr int kMaxTiles = kResKVBytes / (kKTile + kVTile);
  static constexpr int kDK = D / 16;                    // q.k k-steps over d
  static constexpr int kDB = D / 32;                    // 32-row blocks of d
  static constexpr int kKDma = kKTile / 1024 / kResWaves;
  static constexpr int kVDma = kVTile / 1024 / kResWaves;
  static constexpr int kEpiRows = kResEpiBytes / (D * 2);  // output rows per epilogue round
  static_assert(kKDma >= 1 && kVDma >= 1 && kKDma * kResWaves * 1024 == kKTile &&
                kVDma * kResWaves * 1024 == kVTile, "tiles split into whole 1 KB loads per wave");
  static_assert(kEpiRows >= 1 && 32 % kEpiRows == 0, "epilogue rounds");
};

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <typename T>
__device__ __forceinline__ T lds_load(uint32_t addr) {
  return *(const __attribute__((address_space(3))) T*)(uintptr_t)addr;
}

template <int D>
__global__ void __launch_bounds__(kResThreads) attn_resident_kernel(AttnArgs a, int32_t total_tiles) {
  using C = ResCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k_lds[C::kMaxTiles * C::kKTile];
  __shared__ __attribute__((aligned(1024))) char v_lds[C::kMaxTiles * C::kVTile];
  __shared__ __attribute__((aligned(1024))) char e_lds[kResWaves * kResEpiBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // this workgroup's query tiles [it0, it1), tile index = (entry * hc + head) * n_qtiles + tile
  const int64_t nwg = gridDim.x;
  const int it0 = (int)((int64_t)blockIdx.x * total_tiles / nwg);
  const int it1 = (int)((int64_t)(blockIdx.x + 1) * total_tiles / nwg);

  // ---- staging offsets (as in the streaming kernel): wave w fills the 1 KB pieces
  // w*n .. w*n+n-1 of a tile, lane l the bytes [16 l, 16 l + 16) of a piece, i.e.
  // the LDS position that the XOR swizzle gives a logical (row, 16-byte chunk)
  int kdma_row[C::kKDma], kdma_off[C::kKDma], vdma_off[C::kVDma];
#pragma unroll
  for (int i = 0; i < C::kKDma; ++i) {
    const int byte = (wave * C::kKDma + i) * 1024 + lane * 16;
    const int row = byte / C::kKRow;
    const int pc = (byte % C::kKRow) / 16;
    kdma_row[i] = row;
    kdma_off[i] = (pc ^ (row & (C::kKChunks - 1))) * 16;
  }
#pragma unroll
  for (int i = 0; i < C::kVDma; ++i) {
    const int byte = (wave * C::kVDma + i) * 1024 + lane * 16;
    const int row = byte / C::kVRow;
    const int pc = (byte % C::kVRow) / 16;
    vdma_off[i] = row * C::kVRow + (pc ^ ((row >> 1) & 7)) * 16;
  }

  // ---- LDS read addresses: the lane's swizzled offset on top of the array base,
  // held opaque so that the tile, key-block and d-block offsets of every read are
  // immediates (all below 64 KB)
  uint32_t kbase[C::kDK], vbase[4];
  {
    const int kswz = l32 & (C::kKChunks - 1);
    const int vswz = (l32 >> 1) & 7;
#pragma unroll
    for (int kk = 0; kk < C::kDK; ++kk) {
      kbase[kk] = lds_addr(k_lds) + l32 * C::kKRow + (((2 * kk + hl) ^ kswz) << 4);
      asm volatile("" : "+v"(kbase[kk]));
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      vbase[s4] = lds_addr(v_lds) + l32 * C::kVRow + (((2 * s4 + hl) ^ vswz) << 4);
      asm volatile("" : "+v"(vbase[s4]));
    }
  }
  // K fragment of product j (k-step j / 2, key block j % 2) of tile T; V^T
  // fragment of product j (16-key group j / kDB, d block j % kDB) of tile T
  auto kfrag = [&](auto T_, int j) {
    constexpr int T = decltype(T_)::value;
    return lds_load<bf16x8>(kbase[j / 2] + T * C::kKTile + (j % 2) * 32 * C::kKRow);
  };
  auto vfrag = [&](auto T_, int j) {
    constexpr int T = decltype(T_)::value;
    return lds_load<f16x8>(vbase[j / C::kDB] + T * C::kVTile + (j % C::kDB) * 32 * C::kVRow);
  };

  // ---- q of this wave's 32 rows of query tile `it` into the B-operand registers;
  // rows past nq read row nq - 1 (their outputs are not stored)
  bf16x8 qf[C::kDK];
  auto q_addr = [&](int it) {
    const int bh = it / a.n_qtiles;
    const int qt = it - bh * a.n_qtiles;
    const int bat = bh / a.hc;
    const int head = bh - bat * a.hc;
    const int qi = min(qt * kResQ + wave * 32 + l32, a.nq - 1);
    return a.q + bat * a.q_batch + (int64_t)qi * a.q_row + (int64_t)head * a.q_head + 8 * hl;
  };
  auto load_q = [&](const __bf16* qp) {
#pragma unroll
    for (int kk = 0; kk < C::kDK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
  };

  int kv_len = 1, ntiles = 1;
  const float c = a.c;
  // S^T = K * Q^T of tile T, k-steps in order, both key blocks per k-step
  auto scores = [&](auto T_, f32x16 (&s)[2]) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::kDK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(T_, 2 * kk + kb), qf[kk], s[kb], 0, 0, 0);
  };
  // keys past kv_len to -inf when tile T is the last, ragged tile; the limit is
  // opaque so that the comparisons stay inside this (rarely taken) block
  auto mask_last = [&](auto T_, f32x16 (&s)[2]) {
    constexpr int T = decltype(T_)::value;
    if (T == ntiles - 1 && (kv_len & (kBlockN - 1)) != 0) {
      int lim = kv_len - T * kBlockN - 4 * hl;
      asm volatile("" : "+v"(lim));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -__builtin_inff();
    }
  };
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    return mx * c;
  };

  f32x16 o[C::kDB];
  float l_run;
  float lpart[4][2];  // row sums by (pair index mod 4, half), over the whole pass
  // the weights are added one at a time, as the streaming kernel adds them
  // (fma_mix with a register one), so that both kernels give the same bits
  float one = 1.0f;
  asm volatile("" : "+v"(one));
  constexpr int kNS = 2 * C::kDK;     // score products per tile
  constexpr int kNP = 4 * C::kDB;     // weight products per tile
  constexpr int kR = 4;               // LDS fragments read ahead
  constexpr int kPairs = 16;          // float16 weight pairs per lane and tile
  constexpr int kPPG = kPairs / kNS;  // pairs per score product
  static_assert(kNS >= kR && kNP >= kR && kPairs % kNS == 0 && kPairs % kNP == 0, "pipeline shape");

  // weights of pair p of the held scores: x = s*c - m, 2^x, rounded to float16
  auto pair_x = [&](const f32x16 (&s)[2], float nm, int p, float& x0, float& x1) {
    const int s4 = p >> 2, e = p & 3;
    const int r = (s4 & 1) * 8 + 2 * e;
    x0 = __builtin_fmaf(s[s4 >> 1][r], c, nm);
    x1 = __builtin_fmaf(s[s4 >> 1][r + 1], c, nm);
  };
  auto round_pair = [&](float e0, float e1, int p, f16x2 (&hv)[kPairs], u32x4 (&bits)[4]) {
    f16x2 h2;
    h2[0] = (_Float16)e0;
    h2[1] = (_Float16)e1;
    uint32_t u = __builtin_bit_cast(uint32_t, h2);
    asm volatile("" : "+v"(u));  // keeps the weights in their group
    hv[p] = __builtin_bit_cast(f16x2, u);
    bits[p >> 2][p & 3] = u;
  };

  // scores of tile T with the weights of the held scores (of tile T - 1), the
  // steps of each weight pair spread over three consecutive products as in the
  // streaming kernel; leaves the first kR V^T fragments of tile T - 1 in vr
  auto score_phase = [&](auto T_, const f32x16 (&s_cur)[2], f32x16 (&s_next)[2], float mref, f16x8 (&vr)[kR],
                         f16x8 (&pf)[4], f16x2 (&hv)[kPairs]) {
    constexpr int T = decltype(T_)::value;
    const std::integral_constant<int, T - 1> prev{};
    bf16x8 kr[kR];
    u32x4 bits[4];
    s_next[0] = f32x16{};
    s_next[1] = f32x16{};
    const float nm = -mref;
    float xs[kPPG][2], es[kPPG][2];
    auto form_x = [&](int g) {
#pragma unroll
      for (int j = 0; j < kPPG; ++j) {
        pair_x(s_cur, nm, g * kPPG + j, xs[j][0], xs[j][1]);
        asm volatile("" : "+v"(xs[j][0]), "+v"(xs[j][1]));
      }
    };
    auto exp_x = [&]() {
#pragma unroll
      for (int j = 0; j < kPPG; ++j) {
        es[j][0] = __builtin_amdgcn_exp2f(xs[j][0]);
        es[j][1] = __builtin_amdgcn_exp2f(xs[j][1]);
        asm volatile("" : "+v"(es[j][0]), "+v"(es[j][1]));
      }
    };
    auto round_w = [&](int g) {
#pragma unroll
      for (int j = 0; j < kPPG; ++j) round_pair(es[j][0], es[j][1], g * kPPG + j, hv, bits);
    };
#pragma unroll
    for (int j = 0; j < kR; ++j) kr[j] = kfrag(T_, j);
    form_x(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < kNS; ++g) {
      s_next[g % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[g % kR], qf[g / 2], s_next[g % 2], 0, 0, 0);
      if (g + kR < kNS)
        kr[g % kR] = kfrag(T_, g + kR);
      else
        vr[g + kR - kNS] = vfrag(prev, g + kR - kNS);
      if (g > 0) round_w(g - 1);
      exp_x();
      if (g + 1 < kNS) form_x(g + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    round_w(kNS - 1);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) pf[s4] = __builtin_bit_cast(f16x8, bits[s4]);
  };
  // weights of the held scores of the last tile T (no further scores)
  auto weight_phase = [&](auto T_, const f32x16 (&s_cur)[2], float mref, f16x8 (&vr)[kR], f16x8 (&pf)[4],
                          f16x2 (&hv)[kPairs]) {
    u32x4 bits[4];
    const float nm = -mref;
#pragma unroll
    for (int j = 0; j < kR; ++j) vr[j] = vfrag(T_, j);
#pragma unroll
    for (int p = 0; p < kPairs; ++p) {
      float x0, x1;
      pair_x(s_cur, nm, p, x0, x1);
      round_pair(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1), p, hv, bits);
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) pf[s4] = __builtin_bit_cast(f16x8, bits[s4]);
  };
  // O^T += V^T P^T of tile T, the row sums of the rounded weights alongside
  auto product_phase = [&](auto T_, f16x8 (&vr)[kR], const f16x8 (&pf)[4], const f16x2 (&hv)[kPairs]) {
#pragma unroll
    for (int g = 0; g < kNP; ++g) {
      const int s4 = g / C::kDB, db = g % C::kDB;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vr[g % kR], pf[s4], o[db], 0, 0, 0);
      if (g + kR < kNP) vr[g % kR] = vfrag(T_, g + kR);
#pragma unroll
      for (int p = g * kPairs / kNP; p < (g + 1) * kPairs / kNP; ++p) {
        float& l0 = lpart[p & 3][0];
        float& l1 = lpart[p & 3][1];
        l0 = __builtin_fmaf((float)hv[p][0], one, l0);
        l1 = __builtin_fmaf((float)hv[p][1], one, l1);
        asm volatile("" : "+v"(l0), "+v"(l1));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // one pass over the key tiles with reference mref; the scores of tile 0 are in
  // s[0]. Every tile but the last of the array forms the scores of the next array
  // tile, also past ntiles (stale LDS, never used: one tile of discarded products
  // per query tile when the keys do not fill the array, where the kernel waits on
  // memory anyway), so each tile has a single code path. With `qnext` set, the q
  // rows it points to are loaded right after the last score product that runs.
  f32x16 s[2][2];
  auto main_pass = [&](float mref, const __bf16* qnext) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lpart[i][0] = lpart[i][1] = 0.0f;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) o[db] = f32x16{};
    const int last_scores = ntiles == C::kMaxTiles ? ntiles - 2 : ntiles - 1;
    static_for<0, C::kMaxTiles>([&](auto T_) {
      constexpr int T = decltype(T_)::value;
      if (T < ntiles) {
        f16x8 vr[kR];
        f16x8 pf[4];
        f16x2 hv[kPairs];
        if constexpr (T + 1 < C::kMaxTiles) {
          const std::integral_constant<int, T + 1> nxt{};
          score_phase(nxt, s[T & 1], s[(T + 1) & 1], mref, vr, pf, hv);
          mask_last(nxt, s[(T + 1) & 1]);
          if (T == last_scores && qnext) load_q(qnext);
        } else {
          weight_phase(T_, s[T & 1], mref, vr, pf, hv);
        }
        product_phase(T_, vr, pf, hv);
      }
    });
    const float q0 = lpart[0][0] + lpart[0][1], q1 = lpart[1][0] + lpart[1][1];
    const float q2 = lpart[2][0] + lpart[2][1], q3 = lpart[3][0] + lpart[3][1];
    l_run = (q0 + q1) + (q2 + q3);
  };

  const std::integral_constant<int, 0> tile0{};
  int cur_bh = -1;
  if (it0 < it1) load_q(q_addr(it0));
  for (int it = it0; it < it1; ++it) {
    const int bh = it / a.n_qtiles;
    const int qt = it - bh * a.n_qtiles;
    const int bat = bh / a.hc;
    const int head = bh - bat * a.hc;
    if (bh != cur_bh) {
      // every wave is done with the previous head's tiles before they are replaced
      __syncthreads();
      cur_bh = bh;
      kv_len = a.kv_len[bat];
      // at most kMaxTiles (the launcher rejects longer keys): the LDS bound holds anyway
      ntiles = min((kv_len + kBlockN - 1) / kBlockN, C::kMaxTiles);
      const char* kbytes = reinterpret_cast<const char*>(a.k + bat * a.k_batch + (int64_t)head * a.k_head);
      const char* vbytes = reinterpret_cast<const char*>(a.vt + bat * a.vt_batch + (int64_t)head * a.vt_head);
      const int krow_bytes = (int)(a.k_row * 2);
      // K rows at or past kv_len re-read the last valid row (their scores are masked)
      for (int t = 0; t < ntiles; ++t) {
        const char* kt = kbytes + (int64_t)t * kBlockN * krow_bytes;
        const int lim = kv_len - 1 - t * kBlockN;
#pragma unroll
        for (int i = 0; i < C::kKDma; ++i)
          dma16(kt + (uint32_t)(min(kdma_row[i], lim) * krow_bytes + kdma_off[i]),
                lds_addr(k_lds) + t * C::kKTile + (wave_u * C::kKDma + i) * 1024);
        const char* vt = vbytes + (int64_t)t * C::kVTile;
#pragma unroll
        for (int i = 0; i < C::kVDma; ++i)
          dma16(vt + vdma_off[i], lds_addr(v_lds) + t * C::kVTile + (wave_u * C::kVDma + i) * 1024);
      }
      wait_vm<0>();
      barrier_only();
    }
    const __bf16* qnext = it + 1 < it1 ? q_addr(it + 1) : nullptr;

    // reference: the maximum of each row over the first key tile. Rare second
    // attempt: a weight left the float16 range (or the inputs were not finite), and
    // this wave recomputes its rows with the exact row maximum.
    scores(tile0, s[0]);
    mask_last(tile0, s[0]);
    float mref = tile_max(s[0]);
    for (int attempt = 0;; ++attempt) {
      main_pass(mref, attempt == 0 ? qnext : nullptr);
      if (attempt == 1 || !__any(!__builtin_isfinite(l_run))) {
        if (attempt == 1 && qnext) load_q(qnext);
        break;
      }
      load_q(q_addr(it));
      float mx = -__builtin_inff();
      static_for<0, C::kMaxTiles>([&](auto T_) {
        if (decltype(T_)::value < ntiles) {
          scores(T_, s[1]);
          mask_last(T_, s[1]);
          mx = fmaxf(mx, tile_max(s[1]));
        }
      });
      scores(tile0, s[0]);
      mask_last(tile0, s[0]);
      mref = mx;
    }

    // ---- epilogue: normalise, round to bf16, stage kEpiRows rows at a time in this
    // wave's LDS area (the 8-byte pieces of a row XOR-permuted by the row, so that
    // the 32 lanes writing one piece of 32 rows spread over the banks) and store
    // whole rows, 16 bytes per lane. Rows are 256-byte aligned and the permutation
    // is an XOR below 256, so a piece's address is the lane's row base XOR a
    // constant; the bases are opaque so that they are formed here, per query tile,
    // instead of being held in registers across the loop.
    constexpr int kRowBytes = D * 2;
    constexpr int kGran = D / 8;
    constexpr int kRowsPerStore = kWave / kGran;
    static_assert((kRowBytes & (kRowBytes - 1)) == 0 && kResEpiBytes % kRowBytes == 0, "row alignment");
    // 1 / row sum and the power-of-two unscaling of v (exact)
    const VUnscale us = v_unscale(l_run + __shfl_xor(l_run, 32), a.vexp[bh]);
    if (us.rest != 0) {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = __builtin_amdgcn_ldexpf(o[db][r] * us.inv, us.rest);
    } else {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= us.inv;
    }
    const uint32_t stg = lds_addr(e_lds) + wave_u * kResEpiBytes;
    const int q0 = qt * kResQ + wave * 32;
    __bf16* obase = a.out + bat * a.out_batch + (int64_t)head * D;
    const int gi = lane % kGran;
#pragma unroll
    for (int rd = 0; rd < 32 / C::kEpiRows; ++rd) {
      const int row = l32 - rd * C::kEpiRows;
      if (row >= 0 && row < C::kEpiRows) {
        // the lane half picks the odd or even 8-byte piece: folded into the base
        uint32_t wb = (stg + row * kRowBytes + ((2 * (row & (kGran - 1))) << 3)) ^ (uint32_t)(hl << 3);
        asm volatile("" : "+v"(wb));
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)o[db][4 * g + e];
            const int pc = db * 8 + 2 * g;  // 8-byte piece of the row (plus hl)
            *(__attribute__((address_space(3))) bf16x4*)(uintptr_t)(wb ^ (uint32_t)(pc << 3)) = w;
          }
      }
#pragma unroll
      for (int k = 0; k < C::kEpiRows / kRowsPerStore; ++k) {
        const int r = k * kRowsPerStore + lane / kGran;
        uint32_t rb = (stg + r * kRowBytes + ((2 * (r & (kGran - 1))) << 3)) ^ (uint32_t)((2 * gi) << 3);
        asm volatile("" : "+v"(rb));
        const u32x4 v = lds_load<u32x4>(rb);
        const int qi = q0 + rd * C::kEpiRows + r;
        if (qi < a.nq) *reinterpret_cast<u32x4*>(obase + (int64_t)qi * a.hc * D + gi * 8) = v;
      }
    }
  }
}

template <int D>
hipError_t launch_resident_t(AttnArgs a, int cus, hipStream_t s) {
  a.n_qtiles = (a.nq + kResQ - 1) / kResQ;
  const int64_t total = (int64_t)a.n_qtiles * a.hc * a.batch;
  if (total <= 0 || total > 0x7fffffff || cus <= 0) return hipErrorInvalidValue;
  const int nwg = (int)(total < cus ? total : cus);
  hipLaunchKernelGGL((attn_resident_kernel<D>), dim3(nwg), dim3(kResThreads), 0, s, a, (int32_t)total);
  return hipGetLastError();
}

}  // namespace

int resident_max_keys(int head_dim) {
  if (head_dim == 128) return ResCfg<128>::kMaxTiles * kBlockN;
  if (head_dim == 64) return ResCfg<64>::kMaxTiles * kBlockN;
  return 0;
}

int64_t resident_query_tiles(int32_t nq) { return (nq + kResQ - 1) / kResQ; }

hipError_t launch_attn_resident(const AttnArgs& a, int head_dim, int cus, hipStream_t s) {
  if (a.batch <= 0 || a.batch > kMaxBatch || a.hc <= 0 || a.nq <= 0) return hipErrorInvalidValue;
  for (int b = 0; b < a.batch; ++b)
    if (a.kv_len[b] < 1 || a.kv_len[b] > resident_max_keys(head_dim)) return hipErrorInvalidValue;
  if (head_dim == 128) return launch_resident_t<128>(a, cus, s);
  if (head_dim == 64) return launch_resident_t<64>(a, cus, s);
  return hipErrorInvalidValue;
}

}  // namespace vdit

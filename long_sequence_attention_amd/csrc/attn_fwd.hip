// Flash-style attention forward for gfx950 (CDNA4), bf16 q/k, fp16 weights and v.
//
// Work split: one workgroup = WAVES waves = BLOCK_M = WAVES * QB * 32 queries of one
// head (WAVES / 2 * QB * 32 in the block-sparse mode below); it streams all valid
// keys of that head in tiles of 64 keys. K tiles (row-major, from the input or the
// rotated-key workspace) and V^T tiles (prepared in the workspace) reach LDS by
// direct global->LDS loads (global_load_lds_dwordx4): for long key sequences into
// four K and four V^T stages, issued four (K) and two (V^T) iterations ahead; for
// short ones and the block-sparse mode into two of each, so that two workgroups
// share a CU.
//
// Per wave and key tile the scores are formed transposed, S^T = K * Q^T, with
// v_mfma_f32_32x32x16_bf16: the A operand is a 32-key x 16-dim slice of K read
// from LDS, the B operand is the wave's queries held in registers for the whole
// loop. In the 32x32 accumulator layout lane l holds query (l % 32) and 16 of
// its keys, the other 16 in lane l ^ 32. The float16 weights P^T stay in the
// same lanes and serve directly as the B operand of O^T += V^T * P^T
// (v_mfma_f32_32x32x16_f16); the workspace stores V^T with the key order inside
// each group of 16 permuted (bits 2 and 3 of the key index swapped) so that the
// A operand for a lane is one 16-byte LDS read.
//
// Per iteration a wave forms the scores of the next tile while it turns half of
// the held scores into weights, then runs the weight products while it turns the
// other half of the next tile's scores into weights, so both phases carry the same
// vector work. With four stages the two waves sharing a SIMD are kept half an
// iteration apart (one forms scores while the other runs products).
//
// Block-sparse mode (SPARSE): the workgroup is one 64-query tile and visits only
// the key tiles listed for it, in list order. Four waves split it: wave w takes
// queries 32 (w / 2) .. + 31 and keys 32 (w % 2) .. + 31 of every tile, with its
// own softmax reference, row sums and accumulators; the two waves of a query
// block merge their partial results at the end. So two waves share each SIMD,
// as in the dense kernel, although one query tile is only 64 rows.
//
// Softmax: the weights use a fixed reference, the row maximum of the first key
// tile, in the log2 domain (c = scale * log2 e): p = 2^(s*c - m). O is never
// rescaled. If some later score exceeds the reference by more than the float16
// range allows, a weight becomes inf and the row sum non-finite; such rows are
// appended to a retry list of their (entry, head), and a second launch of the
// same kernel (RETRY) recomputes only the listed rows, 256 per workgroup, with
// the exact row maximum (a q.k-only pass for the maximum, then the normal pass,
// where every weight is at most 1). In the block-sparse mode the workgroup
// recomputes its own rows instead. The row sum is taken from the rounded float16
// weights (added one by one in float32), the same values the product uses.
#include "common.hpp"
#include "lds.hpp"

#include <atomic>

namespace vdit {
namespace {

template <int D, int QB, int WAVES, bool QK8 = false, int KS = 1>
struct FwdCfg {
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKSplit = KS;                     // waves sharing the keys of each query row
  static constexpr int kBlockM = kWaves / KS * QB * 32;
  static constexpr int kKRow = QK8 ? D : D * 2;          // bytes per K row in LDS (int8 or bf16)
  static constexpr int kKChunks = kKRow / 16;            // 16-byte chunks per K row
  static constexpr int kVRow = kBlockN * 2;              // bytes per V^T row in LDS
  static constexpr int kKTile = kBlockN * kKRow;         // bytes
  static constexpr int kVTile = D * kVRow;               // bytes
  static constexpr int kKDma = kKTile / 1024 / kWaves;   // 1 KB direct loads per wave per K tile
  static constexpr int kVDma = kVTile / 1024 / kWaves;
  static constexpr int kDK = QK8 ? D / 32 : D / 16;     // q.k MFMA k-steps over d (16 bytes per lane)
  static constexpr int kDB = D / 32;                     // 32-row blocks of d
  static_assert(kKDma >= 1 && kVDma >= 1 && kKDma * kWaves * 1024 == kKTile && kVDma * kWaves * 1024 == kVTile,
                "tiles must split into whole 1 KB direct loads per wave");
};

// NST = LDS stages per operand: 4 (K staged four and V^T two iterations ahead,
// with the wave offset below) for one large workgroup per CU, or 2 (K two and
// V^T one iteration ahead, 64 KB of LDS) so that two smaller workgroups share a
// CU and one computes while the other waits on memory.
// QK8: q.k on int8 codes per block (v_mfma_i32_32x32x32_i8), prepared by the
// quantize pre-pass with the softmax scale folded into q. The integer scores come
// out of the products already readable as floats (offset by a constant, see
// qk_mfma); each tile's weights use c = q scale * k scale * log2 e per lane.
// RETRY: the second launch, over the rows listed by the first: workgroup (entry,
// head, c) takes the listed rows 256 c .. 256 c + 255 (none: it returns at once).
template <int D, int QB, int WAVES, int NST, bool ROPE, bool QK8, bool SPARSE, bool RETRY>
__global__ void __launch_bounds__(WAVES * 64) attn_fwd_kernel(AttnArgs a) {
  constexpr int KS = SPARSE ? 2 : 1;  // waves per query block (key split)
  constexpr int KH = 2 / KS;          // 32-key blocks per wave and tile
  using C = FwdCfg<D, QB, WAVES, QK8, KS>;
  using QFrag = typename std::conditional<QK8, i32x4, bf16x8>::type;
  static_assert(!(QK8 && ROPE), "int8 q.k takes no RoPE");
  static_assert(!SPARSE || (!QK8 && !ROPE && C::kBlockM == 64), "block-sparse: bfloat16, 64-query tiles");
  static_assert(NST == 4 || NST == 2, "stage count");
  static_assert(NST == 2 || WAVES % 2 == 0, "the wave offset pairs waves w and w + WAVES/2");
  static_assert(!(RETRY && SPARSE) && (!RETRY || QB == 1), "row lists: dense, one query block per wave");
  // K and V^T stages, each its own array (not one array indexed by stage) so
  // that the compiler can tell a direct load into one stage from reads of
  // another and does not wait for the direct loads before LDS reads.
  constexpr int kKHi = NST == 4 ? C::kKTile : 1024;  // stages 2, 3 (unused with NST = 2)
  constexpr int kVHi = NST == 4 ? C::kVTile : 1024;
  __shared__ __attribute__((aligned(1024))) char k_st0[C::kKTile];
  __shared__ __attribute__((aligned(1024))) char k_st1[C::kKTile];
  __shared__ __attribute__((aligned(1024))) char k_st2[kKHi];
  __shared__ __attribute__((aligned(1024))) char k_st3[kKHi];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::kVTile];
  __shared__ __attribute__((aligned(1024))) char v_st1[C::kVTile];
  __shared__ __attribute__((aligned(1024))) char v_st2[kVHi];
  __shared__ __attribute__((aligned(1024))) char v_st3[kVHi];
  __shared__ int wg_retry;
  // int8 q.k: k scale of every key tile of this (entry, head), copied in the prologue
  __shared__ float ks_lds[QK8 ? (NST == 4 ? kQK8MaxTiles : kSmallKeys / kBlockN) : 1];
  // block-sparse: the key tiles this workgroup visits (with cube tiles, bits 13-15
  // mark the last cube along t, y and x, whose token counts are fixed)
  __shared__ uint16_t tile_lds[SPARSE ? kVsaMaxKeep : 1];
  // block-sparse cube tiles: the two waves of a query block exchange their references
  __shared__ float ref_lds[SPARSE ? WAVES * 32 : 1];
  // retry launch: the query rows of the chunk in progress (-1 past the list)
  __shared__ int row_lds[RETRY ? C::kBlockM : 1];

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so that
  // each XCD walks a contiguous range of (head, query tile) and its L2 serves the
  // K/V tiles of one head to all its CUs.
  int bh, qtile;
  if constexpr (RETRY) {
    bh = blockIdx.x / a.n_qtiles;
    qtile = blockIdx.x - bh * a.n_qtiles;      // chunk of the row list
  } else {
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    const int xcd = wg & 7;
    const int per = nwg >> 3;
    const int rem = nwg & 7;
    const int id = xcd * per + (xcd < rem ? xcd : rem) + (wg >> 3);
    bh = id / a.n_qtiles;                    // batch entry * hc + local head
    qtile = id - bh * a.n_qtiles;
  }
  const int bat = bh / a.hc;
  const int head = bh - bat * a.hc;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int qw = wave / KS;               // query block of the wave
  const int kblk0 = KS == 2 ? wave & 1 : 0;  // first 32-key block of each tile it takes

  if (tid == 0) wg_retry = 0;

  // retry launch: the rows listed for this (entry, head), chunk qtile of them
  int n_listed = 0;
  if constexpr (RETRY) {
    // written by the attention launch before this one: a plain (scalar) load sees it
    n_listed = a.retry_cnt[2 * bh];
    if (qtile * C::kBlockM >= n_listed) return;  // whole workgroup: nothing listed here
    const int i = qtile * C::kBlockM + tid;
    if (tid < C::kBlockM) row_lds[tid] = i < n_listed ? a.retry_rows[(int64_t)bh * a.nq + i] : -1;
    __syncthreads();
  }
  // block-sparse cube tiles: the query tile is cube qtile
  Cube qcube{};
  if constexpr (SPARSE)
    if (a.cube.on) qcube = cube_at(a.cube, qtile);
  // query row of row r of this wave (-1: none)
  auto row_of = [&](int r) -> int {
    if constexpr (RETRY) {
      return row_lds[qw * QB * 32 + r];
    } else {
      if constexpr (SPARSE) {
        const int slot = qw * QB * 32 + r;
        if (a.cube.on) return slot < qcube.len ? cube_token(a.cube, qcube, slot) : -1;
      }
      return qtile * C::kBlockM + qw * QB * 32 + r;
    }
  };

  // ---- this wave's queries into registers (B operand layout), RoPE fused
  QFrag qf[QB][C::kDK];
  float cq[QB];  // factor of the float scores in the exponent (log2 domain)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = row_of(qb * 32 + l32);
    cq[qb] = a.c;
    if (qi >= 0 && qi < a.nq) {
      if constexpr (QK8) {
        // lane half h holds dims [32 kk + 16 h, 32 kk + 16 h + 16) of k-step kk
        const int8_t* qp = a.qc + bh * a.qc_bh + (int64_t)qi * D + 16 * hl;
#pragma unroll
        for (int kk = 0; kk < C::kDK; ++kk) qf[qb][kk] = *reinterpret_cast<const i32x4*>(qp + 32 * kk);
        cq[qb] = a.qsc[(int64_t)bh * a.nq_blocks + qi / kQuantQ] * a.c;
      } else {
        const __bf16* qp = a.q + bat * a.q_batch + (int64_t)qi * a.q_row + (int64_t)head * a.q_head + 8 * hl;
        int t = 0, y = 0, x = 0;
        if constexpr (ROPE) rope_token_pos(a.rope, qi, t, y, x);
#pragma unroll
        for (int kk = 0; kk < C::kDK; ++kk) {
          bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
          if constexpr (ROPE) v = rope_chunk(a.rope, v, 16 * kk + 8 * hl, t, y, x);
          qf[qb][kk] = v;
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < C::kDK; ++kk) qf[qb][kk] = QFrag{};
    }
  }

  const int kv_len = a.kv_len[bat];
  const int ktiles = (kv_len + kBlockN - 1) / kBlockN;  // key tiles of the entry
  const int ntiles = SPARSE ? a.keep : ktiles;           // key tiles visited
  if constexpr (SPARSE) {
    // tile indices out of range are clamped, so every load stays in bounds
    const int32_t* lst = a.tiles + ((int64_t)bh * a.n_qtiles + qtile) * a.keep;
    static_assert(kVsaMaxTiles <= (1 << 13), "tile indices below bit 13");
    for (int i = tid; i < ntiles; i += C::kThreads) {
      const int j = min(max(lst[i], 0), ktiles - 1);
      const int fl = a.cube.on ? cube_at(a.cube, j).flags : 0;
      tile_lds[i] = (uint16_t)(j | (fl << 13));
    }
    __syncthreads();
  }
  // key tile of visit t; visits past the last one repeat it
  auto tile_of = [&](int t) -> int {
    t = min(t, ntiles - 1);
    if constexpr (SPARSE)
      return tile_lds[t] & 0x1fff;
    else
      return t;
  };
  const char* kbytes = QK8 ? reinterpret_cast<const char*>(a.kc + bh * a.kc_bh)
                           : reinterpret_cast<const char*>(a.k + bat * a.k_batch + (int64_t)head * a.k_head);
  const char* vbytes = reinterpret_cast<const char*>(a.vt + bat * a.vt_batch + (int64_t)head * a.vt_head);
  const int krow_bytes = QK8 ? D : (int)(a.k_row * 2);
  // factor of tile t's float scores in the exponent: c, or with int8 q.k
  // q scale * k scale * log2 e (at least FLT_MIN, so that masked scores stay -inf).
  // The k scales are read from LDS: a global load here would make the compiler
  // wait for every direct load in flight.
  auto tile_c = [&](int t, float (&ct)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if constexpr (QK8)
        ct[qb] = fmaxf(cq[qb] * ks_lds[min(t, ntiles - 1)], 0x1p-126f);
      else
        ct[qb] = cq[qb];
    }
  };

  // ---- direct global -> LDS staging. Wave w fills the 1 KB pieces w*n .. w*n+n-1
  // of a tile; lane l writes bytes [16 l, 16 l + 16) of a piece, i.e. the LDS
  // position (row, physical chunk) that the XOR swizzle assigns to a logical
  // (row, chunk) of the tile, so each lane fetches that logical chunk.
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
  // K rows past kv_len re-read the last valid row (their scores are masked), so
  // no row at or beyond kv_len is ever read; tiles past the last one re-read it.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // byte offsets of the lanes' K chunks inside a full tile (rows unclamped)
  uint32_t kdma_full[C::kKDma];
#pragma unroll
  for (int i = 0; i < C::kKDma; ++i) kdma_full[i] = (uint32_t)(kdma_row[i] * krow_bytes + kdma_off[i]);
  auto dma_k = [&](int t, const char* st) {
    t = tile_of(t);
    const char* kt = kbytes + (int64_t)t * kBlockN * krow_bytes;
    const int lim = kv_len - 1 - t * kBlockN;
    if (lim >= kBlockN - 1) {
#pragma unroll
      for (int i = 0; i < C::kKDma; ++i) dma16(kt + kdma_full[i], lds_addr(st) + (wave_u * C::kKDma + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < C::kKDma; ++i) {
        const int row = min(kdma_row[i], lim);
        dma16(kt + (uint32_t)(row * krow_bytes + kdma_off[i]), lds_addr(st) + (wave_u * C::kKDma + i) * 1024);
      }
    }
  };
  auto dma_v = [&](int t, const char* st) {
    t = tile_of(t);
    const char* vt = vbytes + (int64_t)t * C::kVTile;
#pragma unroll
    for (int i = 0; i < C::kVDma; ++i) dma16(vt + vdma_off[i], lds_addr(st) + (wave_u * C::kVDma + i) * 1024);
  };

  // per-lane LDS read offsets: the XOR swizzle depends only on the lane and the
  // k-step, so the stage base and the 32-row block fold into the immediate offset.
  // voff[g]: the wave's g-th group of 16 keys (groups 2 kblk0 .. of the tile).
  int koff[C::kDK], voff[2 * KH];
  {
    const int kswz = l32 & (C::kKChunks - 1);
    const int vswz = (l32 >> 1) & 7;
#pragma unroll
    for (int kk = 0; kk < C::kDK; ++kk) koff[kk] = l32 * C::kKRow + (((2 * kk + hl) ^ kswz) << 4);
#pragma unroll
    for (int s4 = 0; s4 < 2 * KH; ++s4) voff[s4] = l32 * C::kVRow + (((2 * (s4 + 2 * kblk0) + hl) ^ vswz) << 4);
  }
  // V^T reads address the lowest V^T stage plus the lane's offset, held opaque, so
  // that each read is that register plus an immediate (stage and 32-row block, below
  // 64 KB); folded into one constant the stage base exceeds the 16-bit immediate
  // and costs an OR per read
  const uint32_t v_lo = min(min(lds_addr(v_st0), lds_addr(v_st1)), min(lds_addr(v_st2), lds_addr(v_st3)));
  uint32_t vbase[2 * KH];
#pragma unroll
  for (int s4 = 0; s4 < 2 * KH; ++s4) {
    vbase[s4] = v_lo + voff[s4];
    asm volatile("" : "+v"(vbase[s4]));
  }

  // S^T = K * Q^T for the K tile in `kl`
  // one q.k product: bfloat16, or int8 with the int32 accumulator carried in the
  // bits of the float vector. The int8 accumulators start from the bits of
  // kMagic = 1.5 * 2^23, so that a finished accumulator holding kMagic's bits + s
  // (|s| <= 128 * 127 * 127 < 2^22) reads as the float kMagic + s exactly: no
  // conversion; the weights subtract kMagic * c with the reference, and the tile
  // maximum subtracts kMagic (exactly) before it is scaled.
  constexpr float kMagic = 12582912.0f;
  f32x16 acc0;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = QK8 ? kMagic : 0.0f;
  auto qk_mfma = [](const QFrag& ka, const QFrag& qv, f32x16 acc) -> f32x16 {
    if constexpr (QK8)
      return __builtin_bit_cast(
          f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qv, __builtin_bit_cast(i32x16, acc), 0, 0, 0));
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qv, acc, 0, 0, 0);
  };
  auto scores = [&](const char* kl, f32x16 (&s)[QB][KH]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KH; ++kb) s[qb][kb] = acc0;
#pragma unroll
    for (int kk = 0; kk < C::kDK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < KH; ++kb) {
        const QFrag ka = *reinterpret_cast<const QFrag*>(kl + (kb + kblk0) * 32 * C::kKRow + koff[kk]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = qk_mfma(ka, qf[qb][kk], s[qb][kb]);
      }
    }
  };
  // scores of keys past kv_len to -inf (only the last key tile can hold such keys)
  const bool ragged = (kv_len & (kBlockN - 1)) != 0;
  // (block-sparse: the ragged last tile, or a cube of fewer than 64 tokens)
  auto mask_tail = [&](int t, f32x16 (&s)[QB][KH]) {
    bool masked;
    int nvalid;  // valid keys of the tile visited at t
    if constexpr (SPARSE) {
      nvalid = kBlockN;
      if (t < ntiles) {
        const int e = tile_lds[t];
        nvalid = a.cube.on ? cube_len_of_flags(a.cube, e >> 13) : kv_len - (e & 0x1fff) * kBlockN;
      }
      masked = nvalid < kBlockN;
    } else {
      masked = t == ntiles - 1 && ragged;
      nvalid = kv_len - t * kBlockN;
    }
    if (masked) {
      // the lane's first key offset past the valid keys of the tile; opaque, so the
      // compiler neither executes this block unconditionally with selects nor keeps
      // the 32 comparisons of the last tile alive across the loop (64 scalar
      // registers, which it then spills)
      int lim = nvalid - kblk0 * 32 - 4 * hl;
      asm volatile("" : "+v"(lim));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KH; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[qb][kb][r] = -__builtin_inff();
    }
  };
  // maximum of the scores of each query in the tile (both lane halves), times c
  auto tile_max = [&](const f32x16 (&s)[QB][KH], const float (&ct)[QB], float (&m)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][0][r]);
#pragma unroll
      for (int kb = 1; kb < KH; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if constexpr (QK8) mx -= kMagic;
      m[qb] = mx * ct[qb];
    }
  };

  // O^T accumulators and row sums of the weights
  f32x16 o[QB][C::kDB];
  float l_run[QB];
  // row sums of the rounded weights in eight partials, indexed by (pair index mod 4,
  // half of the pair), accumulated over the whole pass and added up at its end: the
  // two halves of a pair and consecutive pairs go to different partials, so no
  // addition waits on the one before it
  float lpart[QB][4][2];
  // Each rounded weight is added to its partial as fma(w, one, l) with w read as a
  // float16 half of a pair and `one` held in a register, which compiles to
  // v_fma_mix_f32 (one float32 rounding per addition). A v_dot2 of the pair with
  // (1, 1) does the same work in half the instructions, but on this chip each
  // v_dot2 holds up the matrix products about twice as long as two fma_mix do.
  float one = 1.0f;
  asm volatile("" : "+v"(one));  // a register operand, not an inline constant

  // ---- one iteration's matrix and vector work, scheduled by hand. A tile has
  // kNS score products (k-step j/2, key block j%2) and kNP weight products
  // (key step j/kDB, d block j%kDB) per 32 queries. LDS fragments are read kR
  // products ahead into a ring of registers, and each score product is grouped
  // with its share of the softmax of the previous tile (p = 2^(s*c - m) for the
  // reference m, rounded to float16; a weight above the float16 range becomes
  // inf), so a wave has several LDS reads in flight and vector work to issue
  // while its products run. sched_barrier keeps the compiler from regrouping (it
  // otherwise trades the read-ahead for registers and waits on every read); the
  // empty asm statements pin values to their group where the compiler would
  // otherwise sink their computation into a later block. Per accumulator the
  // products run in the order of scores() above.
  constexpr int kNS = KH * C::kDK;
  constexpr int kNP = 2 * KH * C::kDB;
  constexpr int kR = 4;
  constexpr int kPairs = 8 * KH;             // float16 pairs of weights per lane
  static_assert(kNS >= kR && kNP >= kR && kPairs % kNS == 0 && kPairs % kNP == 0, "pipeline shape");
  auto kfrag = [&](const char* kl, int j) {
    return *reinterpret_cast<const QFrag*>(kl + (j % KH + kblk0) * 32 * C::kKRow + koff[j / KH]);
  };
  auto vfrag = [&](const char* vl, int j) {
    const uint32_t addr = vbase[j / C::kDB] + (lds_addr(vl) - v_lo) + (j % C::kDB) * 32 * C::kVRow;
    return *(const __attribute__((address_space(3))) f16x8*)(uintptr_t)addr;
  };
  // scores of the next tile with the weights of the held one; leaves the first
  // kR V^T fragments of the products in `vr`
  // `issue(g)` runs after score product g (the block-sparse mode issues its
  // direct loads there, one per product)
  // SPLIT: the weights of a tile are formed half in the score phase (pairs
  // kPairs/2 ..) and half in the product phase before it (pairs 0 .. kPairs/2 - 1,
  // from the scores just formed), so that the vector work spreads over both
  // phases: one pair per two score products with bfloat16 q.k (SPLIT2), one per
  // score product with int8 q.k, whose score phase has half as many products.
  constexpr bool SPLIT = KH == 2 && kNP == kPairs && (kNS == kPairs || 2 * kNS == kPairs);
  constexpr bool SPLIT2 = SPLIT && kNS == kPairs;
  constexpr int kHalf = kPairs / 2;
  // pairs per score product in the chained form / exp / round pipeline below, and
  // the first pair of the score phase in those units
  constexpr int kPPG = SPLIT2 ? 1 : (SPLIT ? kHalf : kPairs) / kNS;
  constexpr int kG0 = SPLIT ? kHalf / kPPG : 0;
  auto score_phase = [&](const char* k_read, const char* v_read, const f32x16 (&s_cur)[QB][KH],
                         f32x16 (&s_next)[QB][KH], const float (&ccur)[QB], const float (&mref)[QB],
                         f16x8 (&vr)[kR], f16x8 (&pf)[QB][2 * KH], f16x2 (&hv)[QB][kPairs],
                         const u32x4 (&wpre)[QB][KH], auto&& issue) {
    QFrag kr[kR];
    u32x4 bits[QB][2 * KH];
    if constexpr (SPLIT) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int s4 = 0; s4 < KH; ++s4) {
          bits[qb][s4] = wpre[qb][s4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // through a local: a bit cast of a vector element read element 0
            const uint32_t u = wpre[qb][s4][e];
            hv[qb][s4 * 4 + e] = __builtin_bit_cast(f16x2, u);
          }
        }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KH; ++kb) s_next[qb][kb] = acc0;
    // The weights of a pair p take three dependent steps: x = s*c - m (fma), 2^x
    // (v_exp_f32, on the transcendental unit), rounding to float16. They are spread
    // over three consecutive products: group g rounds the pair of group g-1, takes
    // 2^x for its own pair and forms x for the pair of group g+1, so the steps in
    // one group are independent and the transcendental unit works alongside the
    // other vector instructions (which it does; one chained group let them take
    // turns).
    float xs[kPPG][QB][2], es[kPPG][QB][2];
    auto form_x = [&](int g) {
#pragma unroll
      for (int j = 0; j < kPPG; ++j) {
        const int p = g * kPPG + j;
        const int s4 = p >> 2, e = p & 3;
        const int skb = s4 >> 1, r = (s4 & 1) * 8 + 2 * e;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float nm = QK8 ? -__builtin_fmaf(kMagic, ccur[qb], mref[qb]) : -mref[qb];
          xs[j][qb][0] = __builtin_fmaf(s_cur[qb][skb][r], ccur[qb], nm);
          xs[j][qb][1] = __builtin_fmaf(s_cur[qb][skb][r + 1], ccur[qb], nm);
          asm volatile("" : "+v"(xs[j][qb][0]), "+v"(xs[j][qb][1]));  // keeps x in its group
        }
      }
    };
    auto exp_x = [&]() {
#pragma unroll
      for (int j = 0; j < kPPG; ++j)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          es[j][qb][0] = __builtin_amdgcn_exp2f(xs[j][qb][0]);
          es[j][qb][1] = __builtin_amdgcn_exp2f(xs[j][qb][1]);
          asm volatile("" : "+v"(es[j][qb][0]), "+v"(es[j][qb][1]));  // keeps 2^x in its group
        }
    };
    auto round_w = [&](int g) {
#pragma unroll
      for (int j = 0; j < kPPG; ++j) {
        const int p = g * kPPG + j;
        const int s4 = p >> 2, e = p & 3;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          f16x2 h2;
          h2[0] = (_Float16)es[j][qb][0];
          h2[1] = (_Float16)es[j][qb][1];
          uint32_t u = __builtin_bit_cast(uint32_t, h2);
          asm volatile("" : "+v"(u));  // keeps the weights in this group
          hv[qb][p] = __builtin_bit_cast(f16x2, u);
          bits[qb][s4][e] = u;
        }
      }
    };
#pragma unroll
    for (int j = 0; j < kR; ++j) kr[j] = kfrag(k_read, j);
    if constexpr (!SPLIT2) form_x(kG0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < kNS; ++g) {
      const int kk = g / KH, kb = g % KH;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        s_next[qb][kb] = qk_mfma(kr[g % kR], qf[qb][kk], s_next[qb][kb]);
      issue(g);
      if (g + kR < kNS)
        kr[g % kR] = kfrag(k_read, g + kR);
      else
        vr[g + kR - kNS] = vfrag(v_read, g + kR - kNS);
      if constexpr (SPLIT2) {
        static_assert(kNS == 2 * kHalf, "one pair per two score products");
        if (g % 2 == 0) {
          if (g >= 2) round_w(kHalf / kPPG + g / 2 - 1);
          form_x(kHalf / kPPG + g / 2);
        } else {
          exp_x();
        }
      } else {
        if (g > 0) round_w(kG0 + g - 1);
        exp_x();
        if (g + 1 < kNS) form_x(kG0 + g + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    round_w(SPLIT2 ? kHalf / kPPG + kNS / 2 - 1 : kG0 + kNS - 1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s4 = 0; s4 < 2 * KH; ++s4) pf[qb][s4] = __builtin_bit_cast(f16x8, bits[qb][s4]);
  };
  // O^T += V^T P^T; the row sums of the rounded weights (fma_mix into lpart) ride
  // along with the products, which have no other vector work
  // with int8 q.k this also converts the integer scores of the next tile to
  // float, two per product
  auto product_phase = [&](const char* v_read, f16x8 (&vr)[kR], const f16x8 (&pf)[QB][2 * KH],
                           const f16x2 (&hv)[QB][kPairs], f32x16 (&s_next)[QB][KH], const float (&cnext)[QB],
                           const float (&mref)[QB], u32x4 (&wnext)[QB][KH]) {
    // the first half of the next tile's weights, pair i: x at group 2i, 2^x at 2i+1,
    // rounded at 2i+2
    float xs[QB][2], es[QB][2];
    auto form_n = [&](int i) {
      const int s4 = i >> 2, e = i & 3;
      const int skb = s4 >> 1, r = (s4 & 1) * 8 + 2 * e;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float nm = QK8 ? -__builtin_fmaf(kMagic, cnext[qb], mref[qb]) : -mref[qb];
        xs[qb][0] = __builtin_fmaf(s_next[qb][skb][r], cnext[qb], nm);
        xs[qb][1] = __builtin_fmaf(s_next[qb][skb][r + 1], cnext[qb], nm);
        asm volatile("" : "+v"(xs[qb][0]), "+v"(xs[qb][1]));
      }
    };
    auto exp_n = [&]() {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        es[qb][0] = __builtin_amdgcn_exp2f(xs[qb][0]);
        es[qb][1] = __builtin_amdgcn_exp2f(xs[qb][1]);
        asm volatile("" : "+v"(es[qb][0]), "+v"(es[qb][1]));
      }
    };
    auto round_n = [&](int i) {
      const int s4 = i >> 2, e = i & 3;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f16x2 h2;
        h2[0] = (_Float16)es[qb][0];
        h2[1] = (_Float16)es[qb][1];
        uint32_t u = __builtin_bit_cast(uint32_t, h2);
        asm volatile("" : "+v"(u));
        wnext[qb][s4][e] = u;
      }
    };
#pragma unroll
    for (int g = 0; g < kNP; ++g) {
      const int s4 = g / C::kDB, db = g % C::kDB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vr[g % kR], pf[qb][s4], o[qb][db], 0, 0, 0);
      if (g + kR < kNP) vr[g % kR] = vfrag(v_read, g + kR);
#pragma unroll
      for (int p = g * kPairs / kNP; p < (g + 1) * kPairs / kNP; ++p)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float& l0 = lpart[qb][p & 3][0];
          float& l1 = lpart[qb][p & 3][1];
          l0 = __builtin_fmaf((float)hv[qb][p][0], one, l0);
          l1 = __builtin_fmaf((float)hv[qb][p][1], one, l1);
          asm volatile("" : "+v"(l0), "+v"(l1));  // keeps the sums in this group
        }
      if constexpr (SPLIT) {
        static_assert(kNP == 2 * kHalf, "one pair per two weight products");
        if (g % 2 == 0) {
          if (g >= 2) round_n(g / 2 - 1);
          form_n(g / 2);
        } else {
          exp_n();
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SPLIT) round_n(kHalf - 1);
  };
  // the first half of tile 0's weights (before the pipelined pass)
  auto prime_weights = [&](const f32x16 (&s0)[QB][KH], const float (&c0)[QB], const float (&mref)[QB],
                           u32x4 (&w)[QB][KH]) {
#pragma unroll
    for (int i = 0; i < kHalf; ++i) {
      const int s4 = i >> 2, e = i & 3;
      const int skb = s4 >> 1, r = (s4 & 1) * 8 + 2 * e;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float nm = QK8 ? -__builtin_fmaf(kMagic, c0[qb], mref[qb]) : -mref[qb];
        f16x2 h2;
        h2[0] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[qb][skb][r], c0[qb], nm));
        h2[1] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[qb][skb][r + 1], c0[qb], nm));
        w[qb][s4][e] = __builtin_bit_cast(uint32_t, h2);
      }
    }
  };

  // direct loads issued per iteration by one wave
  constexpr int kPerIter = C::kKDma + C::kVDma;

  // Stage the first tiles (K 0..3 and V 0..1, or K 0..1 and V 0 with two
  // stages) and form the scores of tile 0.
  f32x16 s_a[QB][KH], s_b[QB][KH];
  float c_a[QB], c_b[QB];
  auto load_kscales = [&]() {
    if constexpr (QK8) {
      const float* ksrc = a.ksc + (int64_t)bh * a.nk_blocks;
      for (int i = tid; i < ntiles; i += C::kThreads) ks_lds[i] = ksrc[i];
    }
  };
  auto prologue = [&]() {
    load_kscales();
    dma_k(0, k_st0);
    dma_v(0, v_st0);
    dma_k(1, k_st1);
    if constexpr (NST == 4) {
      dma_v(1, v_st1);
      dma_k(2, k_st2);
      dma_k(3, k_st3);
    }
    wait_vm<0>();
    barrier_only();
    scores(k_st0, s_a);
    mask_tail(0, s_a);
    tile_c(0, c_a);
    // every wave has read stage 0 before iteration 0 refills it
    barrier_only();
  };

  // One software-pipelined pass over all key tiles. Iteration t issues the
  // direct loads of V(t+2) and K(t+4), forms the scores of tile t+1 while it
  // turns the held scores of tile t into weights, then adds V^T(t) P^T(t).
  //
  // Waves w and w + WAVES/2 share a SIMD. The lower half passes the iteration's
  // barrier after the products, the upper half between the two phases, so while
  // one wave of a SIMD forms scores and weights (matrix and vector work) the
  // other runs its products (matrix work only): between two barriers the lower
  // half does S(t+1), W(t), P(t) and the upper half P(t-1), S(t+1), W(t).
  // Every wave passes one barrier per iteration.
  //
  // Stages: K(t) in k_st[t % 4], V(t) in v_st[t % 4]. Between two barriers the
  // waves read K(t+1), V(t) and V(t-1) and fill K(t+4) and V(t+2), which go to
  // stages nobody reads then; the barrier closing the interval guarantees V(t+1)
  // and K(t+2) (issued one and two intervals earlier), so only the newer loads
  // stay in flight. Staging indices past the last tile re-stage the last tile,
  // and the last iteration also forms scores it does not use, so the control
  // flow of every iteration is the same.
  //
  // With NST = 2 there is no offset (the two waves of a SIMD belong to different
  // workgroups): iteration t fills K(t+2) and V(t+1) and waits for all of them
  // before its barrier.
  const bool upper = NST == 4 && wave_u >= C::kWaves / 2;
  auto sync = [&]() {
    if constexpr (NST == 4)
      wait_vm<C::kKDma + kPerIter>();
    else
      wait_vm<0>();
    barrier_only();
  };
  // c_cur / c_next: exponent factors of the scores held for tiles t and t+1
  auto step = [&](int t, char* k_read, char* k_fill, char* v_read, char* v_fill, f32x16 (&s_cur)[QB][KH],
                  f32x16 (&s_next)[QB][KH], const float (&c_cur)[QB], float (&c_next)[QB],
                  const float (&mref)[QB], const u32x4 (&w_cur)[QB][KH], u32x4 (&w_next)[QB][KH]) {
    f16x8 vr[kR];
    f16x8 pf[QB][2 * KH];
    f16x2 hv[QB][kPairs];
    if constexpr (NST == 2) {
      // With two stages (short keys, block-sparse) two workgroups per CU stage
      // their own K/V tiles, so the CU's texture path is busy for much of a step:
      // issued back to back, the loads of all waves queue there together and
      // every wave stalls. Here each wave computes its addresses first and spreads
      // its loads evenly over the score products, K (needed first, by the next
      // scores) before V^T.
      constexpr int kLoads = C::kKDma + C::kVDma;
      constexpr int kEvery = kNS / kLoads;
      static_assert(kEvery >= 1 && kEvery * kLoads <= kNS, "at most one direct load per score product");
      const int tk = tile_of(t + NST), tv = tile_of(t + NST / 2);
      const char* kt = kbytes + (int64_t)tk * kBlockN * krow_bytes;
      const int lim = kv_len - 1 - tk * kBlockN;
      const char* vt = vbytes + (int64_t)tv * C::kVTile;
      const char* ga[C::kKDma + C::kVDma];
      if (lim >= kBlockN - 1) {
#pragma unroll
        for (int i = 0; i < C::kKDma; ++i) ga[i] = kt + kdma_full[i];
      } else {
#pragma unroll
        for (int i = 0; i < C::kKDma; ++i) ga[i] = kt + (uint32_t)(min(kdma_row[i], lim) * krow_bytes + kdma_off[i]);
      }
#pragma unroll
      for (int i = 0; i < C::kVDma; ++i) ga[C::kKDma + i] = vt + vdma_off[i];
      score_phase(k_read, v_read, s_cur, s_next, c_cur, mref, vr, pf, hv, w_cur, [&](int g) {
        if (g % kEvery != 0) return;
        const int i = g / kEvery;
        if (i < C::kKDma)
          dma16(ga[i], lds_addr(k_fill) + (wave_u * C::kKDma + i) * 1024);
        else if (i < kLoads)
          dma16(ga[i], lds_addr(v_fill) + (wave_u * C::kVDma + i - C::kKDma) * 1024);
      });
    } else {
      dma_v(t + NST / 2, v_fill);
      dma_k(t + NST, k_fill);
      score_phase(k_read, v_read, s_cur, s_next, c_cur, mref, vr, pf, hv, w_cur, [](int) {});
    }
    if (upper) sync();
    mask_tail(t + 1, s_next);
    tile_c(t + 1, c_next);
    product_phase(v_read, vr, pf, hv, s_next, c_next, mref, w_next);
    if (!upper) sync();
  };
  auto main_pass = [&](const float (&mref)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) lpart[qb][i][0] = lpart[qb][i][1] = 0.0f;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) o[qb][db] = f32x16{};
    }
    u32x4 w_a[QB][KH], w_b[QB][KH];
    if constexpr (SPLIT) prime_weights(s_a, c_a, mref, w_a);
    if constexpr (NST == 4) {
      for (int t = 0; t < ntiles; t += 4) {
        step(t, k_st1, k_st0, v_st0, v_st2, s_a, s_b, c_a, c_b, mref, w_a, w_b);
        if (t + 1 < ntiles) step(t + 1, k_st2, k_st1, v_st1, v_st3, s_b, s_a, c_b, c_a, mref, w_b, w_a);
        if (t + 2 < ntiles) step(t + 2, k_st3, k_st2, v_st2, v_st0, s_a, s_b, c_a, c_b, mref, w_a, w_b);
        if (t + 3 < ntiles) step(t + 3, k_st0, k_st3, v_st3, v_st1, s_b, s_a, c_b, c_a, mref, w_b, w_a);
      }
    } else {
      for (int t = 0; t < ntiles; t += 2) {
        step(t, k_st1, k_st0, v_st0, v_st1, s_a, s_b, c_a, c_b, mref, w_a, w_b);
        if (t + 1 < ntiles) step(t + 1, k_st0, k_st1, v_st1, v_st0, s_b, s_a, c_b, c_a, mref, w_b, w_a);
      }
    }
    // drain the direct loads still in flight before the stages are reused
    wait_vm<0>();
    barrier_only();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float q0 = lpart[qb][0][0] + lpart[qb][0][1], q1 = lpart[qb][1][0] + lpart[qb][1][1];
      const float q2 = lpart[qb][2][0] + lpart[qb][2][1], q3 = lpart[qb][3][0] + lpart[qb][3][1];
      l_run[qb] = (q0 + q1) + (q2 + q3);
    }
  };

  // exact row maximum: a q.k-only pass over every key tile
  auto exact_max = [&](float (&mx)[QB]) {
    // recompute the staging addresses here instead of keeping the prologue's
    // across the main pass (which would cost registers or scratch there)
#pragma unroll
    for (int i = 0; i < C::kKDma; ++i) asm volatile("" : "+v"(kdma_row[i]), "+v"(kdma_off[i]));
#pragma unroll
    for (int i = 0; i < C::kVDma; ++i) asm volatile("" : "+v"(vdma_off[i]));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = -__builtin_inff();
    for (int t = 0; t < ntiles; ++t) {
      dma_k(t, k_st0);
      wait_vm<0>();
      barrier_only();
      f32x16 s[QB][KH];
      scores(k_st0, s);
      mask_tail(t, s);
      float ct[QB], m[QB];
      tile_c(t, ct);
      tile_max(s, ct, m);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = fmaxf(mx[qb], m[qb]);
      __syncthreads();
    }
  };

  // Block-sparse cube tiles: a cube may hold 32 tokens or fewer, so the key half of a
  // tile that one wave of a query block takes can be empty. Both waves then use the
  // maximum over the whole tile (their two halves) as the reference.
  auto share_ref = [&](float (&m)[QB]) {
    if constexpr (SPARSE) {
      if (a.cube.on) {
        if (hl == 0) ref_lds[wave * 32 + l32] = m[0];
        __syncthreads();
        m[0] = fmaxf(m[0], ref_lds[(wave ^ 1) * 32 + l32]);
      }
    }
  };

  // reference of the weights in o and l_run
  float mfin[QB];
  if constexpr (RETRY) {
    // listed rows: the exact row maximum, so no weight exceeds 1
    if constexpr (QK8) {
      load_kscales();
      __syncthreads();
    }
    exact_max(mfin);
    prologue();
    main_pass(mfin);
  } else {
    // ---- reference maximum from the first key tile
    prologue();
    tile_max(s_a, c_a, mfin);
    share_ref(mfin);
    main_pass(mfin);
    // ---- rare path: some weight left the float16 range (a later key scored far
    // above the first tile's maximum) or the inputs were not finite.
    if constexpr (SPARSE) {
      // the whole workgroup recomputes with the exact row maximum
      bool bad = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) bad |= !__builtin_isfinite(l_run[qb]);
      if (__any(bad) && lane == 0) wg_retry = 1;
      __syncthreads();
      if (wg_retry) {
        exact_max(mfin);
        share_ref(mfin);
        prologue();
        main_pass(mfin);
      }
    } else {
      // the rows go to the retry list of this (entry, head); the retry launch
      // recomputes them (and overwrites what the epilogue below stores for them)
      const int qi = row_of(l32);
      const float lt = l_run[0] + __shfl_xor(l_run[0], 32);
      const bool bad = hl == 0 && qi < a.nq && !__builtin_isfinite(lt);
      const uint64_t m = __ballot(bad);
      if (m != 0) {
        int base = 0;
        if (lane == 0) base = atomicAdd(a.retry_cnt + 2 * bh, __popcll(m));
        base = __shfl(base, 0);
        if (bad) a.retry_rows[(int64_t)bh * a.nq + base + __popcll(m & ((uint64_t(1) << lane) - 1))] = qi;
      }
    }
  }

  // ---- key split: the wave with the second key half hands its row sums,
  // references and accumulators to the first through LDS (the stages are free
  // now); the first merges them, p = 2^(s*c - m) from both sides rescaled to the
  // larger reference. A side whose keys were all masked (reference -inf: only a
  // ragged last tile can give it) adds nothing.
  if constexpr (KS == 2) {
    float* xo = reinterpret_cast<float*>(qw == 0 ? k_st0 : v_st0);  // [QB][kDB][16][64 lanes]
    float* xl = reinterpret_cast<float*>(qw == 0 ? k_st1 : v_st1);  // [QB][2][64 lanes]
    if (kblk0 == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        xl[(qb * 2) * 64 + lane] = l_run[qb] + __shfl_xor(l_run[qb], 32);
        xl[(qb * 2 + 1) * 64 + lane] = mfin[qb];
#pragma unroll
        for (int db = 0; db < C::kDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) xo[((qb * C::kDB + db) * 16 + r) * 64 + lane] = o[qb][db][r];
      }
    }
    __syncthreads();
    if (kblk0 == 1) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l0 = l_run[qb] + __shfl_xor(l_run[qb], 32);
      const float l1 = xl[(qb * 2) * 64 + lane];
      const float m0 = mfin[qb];
      const float m1 = xl[(qb * 2 + 1) * 64 + lane];
      const bool v0 = m0 > -__builtin_inff(), v1 = m1 > -__builtin_inff();
      const float mm = fmaxf(v0 ? m0 : -__builtin_inff(), v1 ? m1 : -__builtin_inff());
      const float a0 = v0 ? __builtin_amdgcn_exp2f(m0 - mm) : 0.0f;
      const float a1 = v1 ? __builtin_amdgcn_exp2f(m1 - mm) : 0.0f;
      const float lt = (v0 ? a0 * l0 : 0.0f) + (v1 ? a1 * l1 : 0.0f);
      // the merged weights are those of the reference mm: the epilogue divides by lt
      l_run[qb] = lt;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x1 = xo[((qb * C::kDB + db) * 16 + r) * 64 + lane];
          o[qb][db][r] = (v0 ? a0 * o[qb][db][r] : 0.0f) + (v1 ? a1 * x1 : 0.0f);
        }
    }
  }

  // ---- epilogue: normalise, round to bf16 and store [nq, hc, d]. Each wave stages
  // its 32 rows in LDS (the staging buffers are free now: every wave has passed the
  // last barrier after its last read of them) and writes them back as whole rows, 16
  // bytes per lane: one store instruction covers 64 / (D / 8) contiguous rows instead
  // of 16-byte pieces of 32 rows. Within a row the 16-byte granules are permuted by
  // an XOR with the row index, so that the writes of the accumulator layout spread
  // over the LDS banks.
  static_assert(QB == 1, "one 32-query block per wave");
  // two waves' rows per full-size V^T stage: stages 2 and 3 exist only with NST = 4
  static_assert(KS == 2 || WAVES <= (NST == 4 ? 8 : 4), "epilogue staging needs two waves per V^T stage");
  static_assert(32 * D * 2 * 2 <= C::kVTile, "two waves' rows fit one V^T stage");
  constexpr int kRowBytes = D * 2;
  constexpr int kGran = D / 8;               // 16-byte granules per row
  constexpr int kRowsPerStore = kWave / kGran;
  char* stg;
  if constexpr (KS == 2) {
    stg = qw == 0 ? k_st0 : v_st0;           // this query block's merge buffer
  } else {
    const int pair = wave_u >> 1;
    char* arr = pair == 0 ? v_st0 : pair == 1 ? v_st1 : pair == 2 ? v_st2 : v_st3;
    stg = arr + (wave_u & 1) * 32 * kRowBytes;
  }
  {
    const float lt = KS == 2 ? l_run[0] : l_run[0] + __shfl_xor(l_run[0], 32);
    // 1 / row sum and the power-of-two unscaling of v (exact)
    const VUnscale us = v_unscale(lt, a.vexp[bh]);
    if (us.rest != 0) {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[0][db][r] = __builtin_amdgcn_ldexpf(o[0][db][r] * us.inv, us.rest);
    } else {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[0][db][r] *= us.inv;
    }
    const int swz = 2 * (l32 & (kGran - 1));
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)o[0][db][4 * g + e];
        const int c = db * 8 + 2 * g + hl;     // 8-byte piece of the row
        *reinterpret_cast<bf16x4*>(stg + l32 * kRowBytes + ((c ^ swz) << 3)) = w;
      }
  }
  {
    const int gi = lane % kGran;
#pragma unroll
    for (int k = 0; k < 32 / kRowsPerStore; ++k) {
      const int row = k * kRowsPerStore + lane / kGran;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * kRowBytes + (((2 * gi) ^ (2 * (row & (kGran - 1)))) << 3));
      const int qi = row_of(row);
      if (qi >= 0 && qi < a.nq) {
        __bf16* op = a.out + bat * a.out_batch + ((int64_t)qi * a.hc + head) * D + gi * 8;
        *reinterpret_cast<u32x4*>(op) = v;
      }
    }
  }

  // retry launch: count the rows done; the workgroup that completes the list
  // clears both counters for the next call (the prepare stage clears them too)
  if constexpr (RETRY) {
    if (tid == 0) {
      const int n_done = min(C::kBlockM, n_listed - qtile * C::kBlockM);
      const int before = atomicAdd(a.retry_cnt + 2 * bh + 1, n_done);
      if (before + n_done == n_listed) {
        atomicExch(a.retry_cnt + 2 * bh, 0);
        atomicExch(a.retry_cnt + 2 * bh + 1, 0);
      }
    }
  }
}

// The attention launch and, for the dense modes, the retry launch over the rows
// whose float16 weights overflowed (usually none: its workgroups then only read
// the row count and return), one workgroup per possible chunk of 256 rows.
template <int D, int QB, int WAVES, int NST, bool ROPE, bool QK8, bool SPARSE = false>
hipError_t launch_fwd_t(AttnArgs a, hipStream_t s) {
  using C = FwdCfg<D, QB, WAVES, QK8, SPARSE ? 2 : 1>;
  a.n_qtiles = SPARSE && a.cube.on ? a.cube.n : (a.nq + C::kBlockM - 1) / C::kBlockM;
  const int64_t nbh = (int64_t)a.hc * a.batch;
  const int64_t nwg = (int64_t)a.n_qtiles * nbh;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidValue;
  if (!SPARSE && (!a.retry_cnt || !a.retry_rows)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_kernel<D, QB, WAVES, NST, ROPE, QK8, SPARSE, false>), dim3((unsigned)nwg),
                     dim3(C::kThreads), 0, s, a);
  if constexpr (!SPARSE)
    hipLaunchKernelGGL((attn_fwd_kernel<D, QB, WAVES, NST, ROPE, QK8, false, true>), dim3((unsigned)nwg),
                       dim3(C::kThreads), 0, s, a);
  return hipGetLastError();
}

// compute units of the current device, queried once per device
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The arguments of batch entry b alone (a batch of one).
AttnArgs entry_args(const AttnArgs& a, int b) {
  AttnArgs e = a;
  e.q = a.q + b * a.q_batch;
  e.k = a.k + b * a.k_batch;
  e.vt = a.vt + b * a.vt_batch;
  e.out = a.out + b * a.out_batch;
  e.vexp = a.vexp + (int64_t)b * a.hc;
  e.retry_cnt = a.retry_cnt ? a.retry_cnt + (int64_t)2 * b * a.hc : nullptr;
  e.retry_rows = a.retry_rows ? a.retry_rows + (int64_t)b * a.hc * a.nq : nullptr;
  e.batch = 1;
  for (int i = 0; i < kMaxBatch; ++i) e.kv_len[i] = 0;
  e.kv_len[0] = a.kv_len[b];
  return e;
}

}  // namespace


hipError_t launch_attn_fwd(const AttnArgs& a, int head_dim, bool rope_q, bool qk_int8, hipStream_t s) {
  if (a.batch <= 0 || a.batch > kMaxBatch || a.hc <= 0) return hipErrorInvalidValue;
  int max_len = 0;
  for (int b = 0; b < a.batch; ++b) max_len = a.kv_len[b] > max_len ? a.kv_len[b] : max_len;
  const bool short_keys = max_len <= kSmallKeys;
  if (qk_int8) {
    // the two-stage int8 configuration holds the k scales of short key sequences only
    if (head_dim != 128 || rope_q) return hipErrorInvalidValue;
    return short_keys ? launch_fwd_t<128, 1, 4, 2, false, true>(a, s) : launch_fwd_t<128, 1, 8, 4, false, true>(a, s);
  }
  // A batch that mixes key lengths fitting the LDS array with longer ones (e.g. the
  // two conditionings of guidance with 512 and 226 text tokens): each entry is
  // launched on its own, so that the short ones take the resident kernel. Both
  // kernels compute every row the same way, so the results do not change.
  if (!rope_q && a.batch > 1) {
    const int rmax = resident_max_keys(head_dim);
    bool any_short = false, any_long = false;
    for (int b = 0; b < a.batch; ++b) {
      if (a.kv_len[b] <= rmax)
        any_short = true;
      else
        any_long = true;
    }
    const int cus = device_cus();
    if (any_short && any_long && cus > 0 && resident_query_tiles(a.nq) * a.hc >= cus) {
      for (int b = 0; b < a.batch; ++b) {
        const hipError_t e = launch_attn_fwd(entry_args(a, b), head_dim, rope_q, qk_int8, s);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  // keys and values that fit in LDS, with a query tile for every CU: the resident
  // kernel (one staging of K/V^T per head and workgroup)
  if (!rope_q && max_len <= resident_max_keys(head_dim)) {
    const int cus = device_cus();
    if (cus > 0 && resident_query_tiles(a.nq) * a.hc * a.batch >= cus) return launch_attn_resident(a, head_dim, cus, s);
  }
  // short keys, or too few 256-query workgroups to give every CU one: the
  // 128-query configuration, two workgroups per CU
  const int64_t big_wgs = (int64_t)((a.nq + 255) / 256) * a.hc * a.batch;
  const bool small = short_keys || big_wgs < 256;
  if (head_dim == 128) {
    if (small)
      return rope_q ? launch_fwd_t<128, 1, 4, 2, true, false>(a, s) : launch_fwd_t<128, 1, 4, 2, false, false>(a, s);
    return rope_q ? launch_fwd_t<128, 1, 8, 4, true, false>(a, s) : launch_fwd_t<128, 1, 8, 4, false, false>(a, s);
  }
  if (head_dim == 64) {
    if (small)
      return rope_q ? launch_fwd_t<64, 1, 4, 2, true, false>(a, s) : launch_fwd_t<64, 1, 4, 2, false, false>(a, s);
    return rope_q ? launch_fwd_t<64, 1, 8, 4, true, false>(a, s) : launch_fwd_t<64, 1, 8, 4, false, false>(a, s);
  }
  return hipErrorInvalidValue;
}

// Block-sparse attention: four waves (64 queries = one query tile, keys split in
// halves) per workgroup and two K/V stages, so two workgroups share a CU.
hipError_t launch_attn_sparse(const AttnArgs& a, int head_dim, hipStream_t s) {
  if (a.batch <= 0 || a.batch > kMaxBatch || a.hc <= 0 || !a.tiles || a.keep < 1 || a.keep > kVsaMaxKeep)
    return hipErrorInvalidValue;
  for (int b = 0; b < a.batch; ++b)
    if (a.kv_len[b] < 1 || a.keep > (a.kv_len[b] + kBlockN - 1) / kBlockN) return hipErrorInvalidValue;
  if (head_dim == 128) return launch_fwd_t<128, 1, 4, 2, false, false, true>(a, s);
  if (head_dim == 64) return launch_fwd_t<64, 1, 4, 2, false, false, true>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace vdit

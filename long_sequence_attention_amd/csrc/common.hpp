// Internal definitions shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace vdit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));    // 16 int8 codes
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kBlockN = 64;  // keys per K/V tile

// 3D RoPE geometry shared by the q prologue, the k pre-pass and the index probe.
// Pair p of the head dimension belongs to band 0 (t) for p < pair_h, band 1 (y)
// for pair_h <= p < pair_w, band 2 (x) otherwise; i is its index inside the band.
// cos/sin of band b at position pos and index i sit at tab[off_b + pos * half_b + i].
struct RopeGeom {
  const float2* tab;  // device table (cos, sin)
  int32_t grid_h, grid_w;
  int32_t pair_h, pair_w;          // first pair of the h and w bands
  int32_t half_t, half_h, half_w;  // pairs per band
  int32_t off_h, off_w;            // table offsets of the h and w bands (t band at 0)
};

struct RopeIndex {
  int32_t band, i, pos;
};

__device__ __forceinline__ void rope_token_pos(const RopeGeom& g, int32_t n, int32_t& t, int32_t& y, int32_t& x) {
  const int32_t hw = g.grid_h * g.grid_w;
  t = n / hw;
  const int32_t r = n - t * hw;
  y = r / g.grid_w;
  x = r - y * g.grid_w;
}

__device__ __forceinline__ RopeIndex rope_pair_index(const RopeGeom& g, int32_t p, int32_t t, int32_t y, int32_t x) {
  RopeIndex r;
  if (p < g.pair_h) {
    r.band = 0; r.i = p; r.pos = t;
  } else if (p < g.pair_w) {
    r.band = 1; r.i = p - g.pair_h; r.pos = y;
  } else {
    r.band = 2; r.i = p - g.pair_w; r.pos = x;
  }
  return r;
}

__device__ __forceinline__ float2 rope_cos_sin(const RopeGeom& g, const RopeIndex& r) {
  int32_t idx;
  if (r.band == 0) idx = r.pos * g.half_t + r.i;
  else if (r.band == 1) idx = g.off_h + r.pos * g.half_h + r.i;
  else idx = g.off_w + r.pos * g.half_w + r.i;
  return g.tab[idx];
}

__device__ __forceinline__ float bf16_to_f32(__bf16 v) { return (float)v; }

// Rotate the 8 consecutive elements [d0, d0 + 8) of one token row (4 pairs) and
// round back to bfloat16. Fixed arithmetic: a' = fma(a, c, -(b*s)), b' = fma(a, s, b*c).
__device__ __forceinline__ bf16x8 rope_chunk(const RopeGeom& g, bf16x8 v, int32_t d0, int32_t t, int32_t y, int32_t x) {
  bf16x8 o;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const RopeIndex ri = rope_pair_index(g, (d0 >> 1) + m, t, y, x);
    const float2 cs = rope_cos_sin(g, ri);
    const float a = (float)v[2 * m];
    const float b = (float)v[2 * m + 1];
    const float ra = __builtin_fmaf(a, cs.x, -(b * cs.y));
    const float rb = __builtin_fmaf(a, cs.y, b * cs.x);
    o[2 * m] = (__bf16)ra;
    o[2 * m + 1] = (__bf16)rb;
  }
  return o;
}

// ---------------------------------------------------------------------------
// Launch parameter blocks.
// ---------------------------------------------------------------------------

// Sequences per call (batch entries) whose key lengths travel in the launch arguments.
constexpr int kMaxBatch = 64;

// Blocks of the int8 quantization of q and k: one scale per block of consecutive
// tokens of one (entry, head).
constexpr int kQuantQ = 128;
constexpr int kQuantK = 64;  // equals kBlockN: one k scale per key tile
// Key tiles whose k scales fit the attention kernel's LDS table (int8 q.k).
constexpr int kQK8MaxTiles = 4096;

// Key lengths up to which the attention runs two smaller workgroups per CU: with
// few key tiles per workgroup its prologue and epilogue dominate, and a second
// workgroup on the CU hides them.
constexpr int kSmallKeys = 1024;

// Block-sparse attention over 64-token tiles (one query tile = one workgroup of
// the sparse attention kernel, one key tile = one K/V tile).
constexpr int kVsaMaxTiles = 8192;  // key tiles one selection can rank (32 keys per thread of the select kernel)
constexpr int kVsaMaxKeep = 4096;   // kept tiles per query tile (the attention kernel's LDS list)

// Block-sparse tiles as 4 x 4 x 4 cubes of a (T, H, W) latent grid (token index
// (t H + y) W + x). Cube j = (ct, cy, cx), numbered with cx fastest, holds the
// tokens with t / 4 = ct, y / 4 = cy, x / 4 = cx in ascending order; the last cube
// along a side that is not a multiple of 4 is thinner, so a cube holds 1 to 64
// tokens. Slot s of a cube (s < its token count) is its s-th token; in the
// workspace a cube occupies one 64-key tile whose slots past the count are zero.
constexpr int kCube = 4;
struct CubeGeom {
  int32_t on;            // 0: tiles are runs of 64 consecutive tokens
  int32_t t, h, w;       // grid sides
  int32_t nct, ncy, ncx; // cubes along each side
  int32_t n;             // cubes, nct * ncy * ncx (at most kVsaMaxTiles)
};

struct Cube {
  int32_t tok0;          // token of the cube's first slot
  int32_t et, ey, ex;    // extent along t, y and x (1..4)
  int32_t len;           // tokens, et * ey * ex
  int32_t flags;         // bit 0/1/2: the last cube along t / y / x
};

__host__ __device__ __forceinline__ Cube cube_at(const CubeGeom& g, int j) {
  const int nyx = g.ncy * g.ncx;
  const int ct = j / nyx;
  const int r = j - ct * nyx;
  const int cy = r / g.ncx;
  const int cx = r - cy * g.ncx;
  Cube c;
  const int rt = g.t - kCube * ct, ry = g.h - kCube * cy, rx = g.w - kCube * cx;
  c.et = rt < kCube ? rt : kCube;
  c.ey = ry < kCube ? ry : kCube;
  c.ex = rx < kCube ? rx : kCube;
  c.len = c.et * c.ey * c.ex;
  c.tok0 = (kCube * ct * g.h + kCube * cy) * g.w + kCube * cx;
  c.flags = (ct == g.nct - 1 ? 1 : 0) | (cy == g.ncy - 1 ? 2 : 0) | (cx == g.ncx - 1 ? 4 : 0);
  return c;
}

// Token of slot s (< c.len) of cube c: slots run x fastest, then y, then t.
__host__ __device__ __forceinline__ int cube_token(const CubeGeom& g, const Cube& c, int s) {
  const int exy = c.ex * c.ey;
  const int dt = s / exy;
  const int r = s - dt * exy;
  const int dy = r / c.ex;
  const int dx = r - dy * c.ex;
  return c.tok0 + (dt * g.h + dy) * g.w + dx;
}

// Token count of a cube from its flags (the extents of the last cubes are fixed).
__host__ __device__ __forceinline__ int cube_len_of_flags(const CubeGeom& g, int flags) {
  const int et = (flags & 1) ? g.t - kCube * (g.nct - 1) : kCube;
  const int ey = (flags & 2) ? g.h - kCube * (g.ncy - 1) : kCube;
  const int ex = (flags & 4) ? g.w - kCube * (g.ncx - 1) : kCube;
  return et * ey * ex;
}

// v is converted to float16 for the weighted sum after scaling by a power of two
// 2^e per (entry, head), chosen from max |v| over the valid keys so that the
// largest value lands in [2^14, 2^15): every bfloat16 value within 2^29 of the
// maximum is then a normal float16 and converts exactly, and nothing overflows.
// The epilogues multiply by 2^-e, which undoes the scaling exactly (a power of
// two commutes with rounding). max |v| is reduced in two steps: kVParts partial
// maxima per (entry, head), then each prepare workgroup combines them.
constexpr int kVParts = 64;
constexpr int kVExpMin = -113;  // bfloat16's largest finite value still lands below 2^15
constexpr int kVExpMax = 160;   // below bfloat16's smallest subnormal
// The epilogue folds min(e, kVExpFold) into 1 / row sum (which stays a normal float:
// the row sum is at most 2^47) and applies the rest of e to each output value.
constexpr int kVExpFold = 64;

// Exponent e of the scaling for a maximum |v| of `amax` (0, inf or NaN: e = 0).
__device__ __forceinline__ int v_scale_exp(float amax) {
  if (!(amax > 0.0f) || amax > 3.4028235e38f) return 0;
  const int e = 15 - __builtin_amdgcn_frexp_expf(amax);  // amax = f * 2^ex, 0.5 <= f < 1
  return e < kVExpMin ? kVExpMin : (e > kVExpMax ? kVExpMax : e);
}

// Epilogue factors undoing the scaling 2^e of v: out = ldexp(o * inv, rest), with
// inv = 2^-min(e, kVExpFold) / row sum and rest = min(e, kVExpFold) - e (0 unless v
// was below about 2^-49, so the per-value ldexp is skipped).
struct VUnscale {
  float inv;
  int rest;
};
__device__ __forceinline__ VUnscale v_unscale(float row_sum, int e) {
  const int fold = e < kVExpFold ? e : kVExpFold;
  return VUnscale{__builtin_amdgcn_ldexpf(1.0f / row_sum, -fold), fold - e};
}

// Element offsets of batch entry b are b * (the *_batch stride) on top of those below.
struct AttnArgs {
  const __bf16* q;       // q of head `head_begin`, token 0, entry 0
  int64_t q_row;         // elements between consecutive tokens of q
  int64_t q_batch;       // elements between batch entries of q
  const __bf16* k;       // k of local head 0, key 0 (input or rotated workspace copy)
  int64_t k_row;         // elements between consecutive keys
  int64_t k_head;        // elements between consecutive local heads of k
  int64_t k_batch;
  const _Float16* vt;    // transposed float16 v in the workspace, local head 0
  int64_t vt_head;       // elements between heads of vt
  int64_t vt_batch;
  __bf16* out;           // [B, nq, hc, d]
  int64_t out_batch;
  int32_t nq;
  int32_t hc;            // heads in the share
  int32_t n_qtiles;      // query tiles per head
  int32_t batch;         // B
  float c;               // scale * log2(e)
  int32_t q_head;        // elements between consecutive heads of q (= d)
  RopeGeom rope;
  // int8 q.k (workspace, laid out per (entry, head) = bh): codes [bh][tokens][d],
  // scales [bh][blocks]
  const int8_t* qc;      // q codes (q already multiplied by the softmax scale)
  const int8_t* kc;      // k codes, [bh][nk_pad][d]
  int64_t qc_bh;         // elements between (entry, head) slices of qc
  int64_t kc_bh;
  const float* qsc;      // q scales, [bh][nq_blocks]
  const float* ksc;      // k scales, [bh][nk_pad / 64]
  int32_t nq_blocks;
  int32_t nk_blocks;
  // block-sparse attention: key tiles kept by each (entry, head, query tile),
  // [bh][n_qtiles][keep], ascending
  const int32_t* tiles;
  int32_t keep;
  const int32_t* vexp;   // [bh]: v was scaled by 2^vexp before the float16 conversion
  // rows whose float16 weights overflowed, per (entry, head): counters [bh][2]
  // (rows listed, rows redone; zero between calls) and the rows [bh][nq]
  int32_t* retry_cnt;
  int32_t* retry_rows;
  int32_t kv_len[kMaxBatch];  // valid keys of each entry
  // block-sparse tiles as latent-grid cubes: q rows are mapped through the cubes, k is
  // the cube-ordered copy in the workspace and kv_len counts its slots
  CubeGeom cube;
};

struct QuantArgs {
  const __bf16* q;       // q of head `head_begin`, token 0, entry 0
  const __bf16* k;
  int64_t q_row, k_row;  // elements between consecutive tokens
  int64_t q_batch, k_batch;
  int64_t head;          // elements between consecutive heads (= d)
  int8_t* qc;
  int8_t* kc;
  int64_t qc_bh, kc_bh;
  float* qsc;
  float* ksc;
  int32_t nq;
  int32_t nq_blocks;     // ceil(nq / 128)
  int32_t nk_blocks;     // blocks of the workspace (nk_pad / 64)
  int32_t hc;
  int32_t batch;
  float sm_scale;        // multiplies q before quantization
  int32_t kv_len[kMaxBatch];
};

struct PrepArgs {
  const __bf16* k;       // k of head `head_begin`, key 0, entry 0
  const __bf16* v;       // v of head `head_begin`, key 0, entry 0
  int64_t kv_row;        // elements between consecutive keys
  int64_t kv_head;       // elements between consecutive heads (= d)
  int64_t kv_batch;      // elements between batch entries of k and v
  _Float16* vt;          // workspace vt, local head 0
  int64_t vt_head;
  __bf16* kr;            // workspace rotated k, local head 0 (nullptr without RoPE)
  int64_t kr_head;
  int32_t n_ktiles;      // ceil(max_b kv_len[b] / 64)
  int32_t hc;
  int32_t batch;
  RopeGeom rope;
  float* vpart;          // [bh][kVParts] partial maxima of |v|
  int32_t* vexp;         // [bh] exponent of the v scaling (written by key tile 0)
  int32_t* retry_cnt;    // [bh][2] retry counters of the attention launch, cleared by key tile 0
  // latent-grid cubes: key tile j of V^T (and of the k copy in kr) holds cube j's
  // tokens, n_ktiles = cubes
  CubeGeom cube;
  int32_t kv_len[kMaxBatch];
};

// Tile means of q or k for the block-sparse selection: float32 [bh][tiles][d].
struct VsaMeanArgs {
  const __bf16* x;  // head `head_begin`, token 0, entry 0
  int64_t row;      // elements between consecutive tokens
  int64_t batch;    // elements between batch entries
  float* mean;
  int32_t n;        // tokens
  int32_t tiles;    // ceil(n / 64), or the cubes
  int32_t hc;
  int32_t bh;       // entries * hc
  CubeGeom cube;    // on: tile j is cube j
};

// Coarse scores [bh][tq][tk] of the tile means, and the kept tiles [bh][tq][keep].
struct VsaSelectArgs {
  const float* qm;  // [bh][tq][d]
  const float* km;  // [bh][tk][d]
  float* s;         // [bh][tq][tk]
  int32_t* tiles;   // [bh][tq][keep]
  int32_t tq, tk, keep, d, bh;
};

// Host-side launchers (defined in the kernel translation units).
hipError_t launch_attn_fwd(const AttnArgs& a, int head_dim, bool rope_q, bool qk_int8, hipStream_t s);
hipError_t launch_attn_sparse(const AttnArgs& a, int head_dim, hipStream_t s);
// Keys and values resident in LDS (short key sequences): the longest key length
// it takes for a head dimension (0 if none), its query tiles per head, and the
// launch on a persistent grid of at most `cus` workgroups.
int resident_max_keys(int head_dim);
int64_t resident_query_tiles(int32_t nq);
hipError_t launch_attn_resident(const AttnArgs& a, int head_dim, int cus, hipStream_t s);
hipError_t launch_vsa_means(const VsaMeanArgs& a, int head_dim, hipStream_t s);
hipError_t launch_vsa_select(const VsaSelectArgs& a, hipStream_t s);
hipError_t launch_prepare(const PrepArgs& a, int head_dim, bool rope_k, hipStream_t s);
hipError_t launch_quantize(const QuantArgs& a, int head_dim, hipStream_t s);
hipError_t launch_pack(const void* src, void* dst, int64_t n, int32_t ht, int32_t d, int32_t groups,
                       bool unpack, hipStream_t s);
hipError_t launch_rope_probe(const RopeGeom& g, int32_t nq, int32_t head_dim, int32_t* out, hipStream_t s);

}  // namespace vdit

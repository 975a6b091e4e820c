// C-ABI entry points: validation, plan, RoPE tables and launches.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "common.hpp"
#include "entry.hpp"
#include "vdit_attn.h"

struct vdit_attn {
  vdit_attn_desc_t desc;  // batch normalised to >= 1
  float scale;
  float c;             // scale * log2(e)
  int device;
  int64_t nk_pad;      // keys rounded up to the key tile
  // block-sparse tiles as latent-grid cubes (vsa_cubes): one 64-slot tile per cube
  vdit::CubeGeom cube;
  int64_t vt_slots;    // key slots per (entry, head) of the V^T and k-copy regions
  size_t ws_vt_off, ws_vt_bytes;
  size_t ws_kr_off, ws_kr_bytes;
  // int8 q.k: codes and scales per (entry, head)
  int64_t nq_pad;      // queries rounded up to the q quantization block
  size_t ws_qc_off, ws_kc_off, ws_qs_off, ws_ks_off;
  // range of v per (entry, head): partial maxima and the exponent of its scaling
  size_t ws_vpart_off, ws_vexp_off;
  // rows whose float16 weights overflowed: counters and row lists per (entry, head)
  size_t ws_rcnt_off, ws_rrows_off;
  size_t ws_total;
  float2* rope_tab;    // device (cos, sin) table, or nullptr
  vdit::RopeGeom geom;
};

namespace {

// Live handles, so that a stale or foreign pointer (e.g. a second destroy) is
// rejected without touching freed memory.
std::mutex g_live_mu;
std::unordered_set<const vdit_attn*>& live_handles() {
  static std::unordered_set<const vdit_attn*> s;
  return s;
}

bool is_live(const vdit_attn* h) {
  if (!h) return false;
  std::lock_guard<std::mutex> lk(g_live_mu);
  return live_handles().count(h) != 0;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

vdit_status_t validate_desc(const vdit_attn_desc_t& d) {
  if (d.batch < 0) return VDIT_ERR_INVALID_ARG;
  if (d.head_dim != 64 && d.head_dim != 128) return VDIT_ERR_UNSUPPORTED;
  if (d.nq < 1 || d.nk < 1 || d.heads_total < 1) return VDIT_ERR_INVALID_ARG;
  if (d.layout != VDIT_LAYOUT_NHD && d.layout != VDIT_LAYOUT_N3HD) return VDIT_ERR_INVALID_ARG;
  if (d.layout == VDIT_LAYOUT_N3HD && d.nq != d.nk) return VDIT_ERR_INVALID_ARG;
  if (d.head_begin < 0 || d.head_count < 1 || (int64_t)d.head_begin + d.head_count > d.heads_total)
    return VDIT_ERR_INVALID_ARG;
  const int64_t batch = d.batch > 0 ? d.batch : 1;
  if (batch > vdit::kMaxBatch || (int64_t)d.head_count * batch > 65535) return VDIT_ERR_UNSUPPORTED;
  if (std::isnan(d.scale) || std::isinf(d.scale)) return VDIT_ERR_INVALID_ARG;
  if (d.use_key_mask != 0 && d.use_key_mask != 1) return VDIT_ERR_INVALID_ARG;
  if (d.use_rope != 0 && d.use_rope != 1) return VDIT_ERR_INVALID_ARG;
  if (d.qk_int8 != 0 && d.qk_int8 != 1) return VDIT_ERR_INVALID_ARG;
  if (d.qk_int8 && (d.head_dim != 128 || d.use_rope || d.nk > vdit::kQK8MaxTiles * vdit::kBlockN))
    return VDIT_ERR_UNSUPPORTED;
  // element offsets are 64-bit in the kernels; keep every tensor below 2^60 elements
  const int64_t row = (int64_t)d.heads_total * d.head_dim * (d.layout == VDIT_LAYOUT_N3HD ? 3 : 1);
  const int64_t nmax = d.nq > d.nk ? d.nq : d.nk;
  if (row > (int64_t(1) << 40) || batch * nmax * row > (int64_t(1) << 60)) return VDIT_ERR_INVALID_ARG;
  // the kernels address a 64-key tile's rows with 32-bit byte offsets (row * stride * 2)
  if (int64_t(vdit::kBlockN) * row * 2 >= (int64_t(1) << 31)) return VDIT_ERR_UNSUPPORTED;
  if (d.vsa_cubes != 0 && d.vsa_cubes != 1) return VDIT_ERR_INVALID_ARG;
  if (d.vsa_cubes) {
    if (d.nq != d.nk) return VDIT_ERR_INVALID_ARG;
    if (d.grid_t < 1 || d.grid_h < 1 || d.grid_w < 1) return VDIT_ERR_INVALID_ARG;
    if ((int64_t)d.grid_t * d.grid_h * d.grid_w != d.nq) return VDIT_ERR_INVALID_ARG;
    const int64_t cubes = (int64_t)((d.grid_t + 3) / 4) * ((d.grid_h + 3) / 4) * ((d.grid_w + 3) / 4);
    if (cubes > vdit::kVsaMaxTiles) return VDIT_ERR_UNSUPPORTED;
  }
  if (d.use_rope) {
    if (d.nq != d.nk) return VDIT_ERR_INVALID_ARG;
    if (d.grid_t < 1 || d.grid_h < 1 || d.grid_w < 1) return VDIT_ERR_INVALID_ARG;
    if ((int64_t)d.grid_t * d.grid_h * d.grid_w != d.nq) return VDIT_ERR_INVALID_ARG;
    const int32_t bt = d.rope_dim_t, bh = d.rope_dim_h, bw = d.rope_dim_w;
    if (bt < 2 || bh < 2 || bw < 2 || (bt | bh | bw) & 1) return VDIT_ERR_INVALID_ARG;
    if ((int64_t)bt + bh + bw != d.head_dim) return VDIT_ERR_INVALID_ARG;
    if (!(d.rope_base > 0.0) || std::isinf(d.rope_base)) return VDIT_ERR_INVALID_ARG;
  }
  return VDIT_OK;
}

// cos/sin of theta = pos * base^(-2i/D) for every band position and pair index,
// computed in double precision and rounded to float.
void build_rope_table(const vdit_attn_desc_t& d, std::vector<float2>& tab, vdit::RopeGeom& g) {
  const int32_t dims[3] = {d.rope_dim_t, d.rope_dim_h, d.rope_dim_w};
  const int32_t npos[3] = {d.grid_t, d.grid_h, d.grid_w};
  int32_t off[3];
  int64_t total = 0;
  for (int b = 0; b < 3; ++b) {
    off[b] = (int32_t)total;
    total += (int64_t)npos[b] * (dims[b] / 2);
  }
  tab.assign((size_t)total, float2{0.f, 0.f});
  for (int b = 0; b < 3; ++b) {
    const int32_t half = dims[b] / 2;
    for (int32_t pos = 0; pos < npos[b]; ++pos)
      for (int32_t i = 0; i < half; ++i) {
        const double inv_freq = std::pow(d.rope_base, -2.0 * (double)i / (double)dims[b]);
        const double theta = (double)pos * inv_freq;
        tab[(size_t)off[b] + (size_t)pos * half + i] = float2{(float)std::cos(theta), (float)std::sin(theta)};
      }
  }
  g.grid_h = d.grid_h;
  g.grid_w = d.grid_w;
  g.half_t = dims[0] / 2;
  g.half_h = dims[1] / 2;
  g.half_w = dims[2] / 2;
  g.pair_h = g.half_t;
  g.pair_w = g.half_t + g.half_h;
  g.off_h = off[1];
  g.off_w = off[2];
}

struct Inputs {
  const __bf16 *q, *k, *v;  // pointing at head_begin, token 0, batch entry 0
  int64_t q_row, kv_row;
  int64_t q_batch, kv_batch;  // elements between batch entries
  size_t q_bytes, k_bytes, v_bytes;  // extents (all entries) for the overlap checks
  const void *q_base, *k_base, *v_base;
};

vdit_status_t resolve_inputs(const vdit_attn& h, const void* q, const void* k, const void* v, Inputs& in) {
  const vdit_attn_desc_t& d = h.desc;
  const int64_t hd = (int64_t)d.heads_total * d.head_dim;
  if (!q) return VDIT_ERR_INVALID_ARG;
  if (d.layout == VDIT_LAYOUT_N3HD) {
    if (k || v) return VDIT_ERR_INVALID_ARG;
    if (!aligned16(q)) return VDIT_ERR_ALIGNMENT;
    const __bf16* base = static_cast<const __bf16*>(q) + (int64_t)d.head_begin * d.head_dim;
    in.q = base;
    in.k = base + hd;
    in.v = base + 2 * hd;
    in.q_row = in.kv_row = 3 * hd;
    in.q_batch = in.kv_batch = (int64_t)d.nq * 3 * hd;
    in.q_bytes = (size_t)d.batch * d.nq * 3 * hd * 2;
    in.k_bytes = in.v_bytes = 0;
    in.q_base = q;
    in.k_base = in.v_base = nullptr;
  } else {
    if (!k || !v) return VDIT_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return VDIT_ERR_ALIGNMENT;
    const int64_t off = (int64_t)d.head_begin * d.head_dim;
    in.q = static_cast<const __bf16*>(q) + off;
    in.k = static_cast<const __bf16*>(k) + off;
    in.v = static_cast<const __bf16*>(v) + off;
    in.q_row = in.kv_row = hd;
    in.q_batch = (int64_t)d.nq * hd;
    in.kv_batch = (int64_t)d.nk * hd;
    in.q_bytes = (size_t)d.batch * d.nq * hd * 2;
    in.k_bytes = in.v_bytes = (size_t)d.batch * d.nk * hd * 2;
    in.q_base = q;
    in.k_base = k;
    in.v_base = v;
  }
  return VDIT_OK;
}

// Valid key count of every batch entry: from key_lens (B values) when given, else
// key_len for all; both are used only with the key mask.
struct KeyLens {
  int32_t len[vdit::kMaxBatch];
  int32_t max;
};

vdit_status_t resolve_lens(const vdit_attn& h, bool per_entry, int32_t key_len, const int32_t* key_lens,
                           KeyLens& kl) {
  const vdit_attn_desc_t& d = h.desc;
  kl.max = 0;
  for (int32_t b = 0; b < vdit::kMaxBatch; ++b) kl.len[b] = 0;
  if (d.use_key_mask && per_entry && !key_lens) return VDIT_ERR_INVALID_ARG;
  for (int32_t b = 0; b < d.batch; ++b) {
    int32_t L = d.nk;
    if (d.use_key_mask) {
      L = per_entry ? key_lens[b] : key_len;
      if (L < 1 || L > d.nk) return VDIT_ERR_INVALID_ARG;
    }
    kl.len[b] = L;
    if (L > kl.max) kl.max = L;
  }
  return VDIT_OK;
}

vdit_status_t check_call(const vdit_attn& h, void* workspace, size_t ws_bytes) {
  if (!workspace || ws_bytes < h.ws_total) return VDIT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return VDIT_ERR_ALIGNMENT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h.device) return VDIT_ERR_DEVICE;
  return VDIT_OK;
}

// cubes: V^T and the k copy in cube order (block-sparse attention over cube tiles)
vdit_status_t do_prepare(const vdit_attn& h, const Inputs& in, const KeyLens& kl, void* ws, hipStream_t s,
                         bool cubes = false) {
  const vdit_attn_desc_t& d = h.desc;
  vdit::PrepArgs a{};
  a.k = in.k;
  a.v = in.v;
  a.kv_row = in.kv_row;
  a.kv_head = d.head_dim;
  a.kv_batch = in.kv_batch;
  a.vt = reinterpret_cast<_Float16*>(static_cast<char*>(ws) + h.ws_vt_off);
  a.vt_head = h.nk_pad * d.head_dim;
  a.kr = d.use_rope ? reinterpret_cast<__bf16*>(static_cast<char*>(ws) + h.ws_kr_off) : nullptr;
  a.kr_head = h.nk_pad * d.head_dim;
  a.n_ktiles = (kl.max + vdit::kBlockN - 1) / vdit::kBlockN;
  a.hc = d.head_count;
  a.batch = d.batch;
  a.rope = h.geom;
  a.vpart = reinterpret_cast<float*>(static_cast<char*>(ws) + h.ws_vpart_off);
  a.vexp = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + h.ws_vexp_off);
  a.retry_cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + h.ws_rcnt_off);
  for (int32_t b = 0; b < vdit::kMaxBatch; ++b) a.kv_len[b] = kl.len[b];
  if (cubes) {
    a.cube = h.cube;
    a.n_ktiles = h.cube.n;
    a.vt_head = h.vt_slots * d.head_dim;
    a.kr = reinterpret_cast<__bf16*>(static_cast<char*>(ws) + h.ws_kr_off);
    a.kr_head = h.vt_slots * d.head_dim;
  }
  if (vdit::launch_prepare(a, d.head_dim, d.use_rope != 0 && !cubes, s) != hipSuccess) return VDIT_ERR_DEVICE;
  if (d.qk_int8) {
    char* w = static_cast<char*>(ws);
    vdit::QuantArgs qa{};
    qa.q = in.q;
    qa.k = in.k;
    qa.q_row = in.q_row;
    qa.k_row = in.kv_row;
    qa.q_batch = in.q_batch;
    qa.k_batch = in.kv_batch;
    qa.head = d.head_dim;
    qa.qc = reinterpret_cast<int8_t*>(w + h.ws_qc_off);
    qa.kc = reinterpret_cast<int8_t*>(w + h.ws_kc_off);
    qa.qc_bh = h.nq_pad * d.head_dim;
    qa.kc_bh = h.nk_pad * d.head_dim;
    qa.qsc = reinterpret_cast<float*>(w + h.ws_qs_off);
    qa.ksc = reinterpret_cast<float*>(w + h.ws_ks_off);
    qa.nq = d.nq;
    qa.nq_blocks = (int32_t)(h.nq_pad / vdit::kQuantQ);
    qa.nk_blocks = (int32_t)(h.nk_pad / vdit::kQuantK);
    qa.hc = d.head_count;
    qa.batch = d.batch;
    qa.sm_scale = h.scale;
    for (int32_t b = 0; b < vdit::kMaxBatch; ++b) qa.kv_len[b] = kl.len[b];
    if (vdit::launch_quantize(qa, d.head_dim, s) != hipSuccess) return VDIT_ERR_DEVICE;
  }
  return VDIT_OK;
}

vdit_status_t do_attend(const vdit_attn& h, const Inputs& in, const KeyLens& kl, void* out, void* ws,
                        hipStream_t s) {
  const vdit_attn_desc_t& d = h.desc;
  vdit::AttnArgs a{};
  a.q = in.q;
  a.q_row = in.q_row;
  a.q_head = d.head_dim;
  a.q_batch = in.q_batch;
  if (d.use_rope) {
    a.k = reinterpret_cast<const __bf16*>(static_cast<const char*>(ws) + h.ws_kr_off);
    a.k_row = d.head_dim;
    a.k_head = h.nk_pad * d.head_dim;
    a.k_batch = a.k_head * d.head_count;
  } else {
    a.k = in.k;
    a.k_row = in.kv_row;
    a.k_head = d.head_dim;
    a.k_batch = in.kv_batch;
  }
  a.vt = reinterpret_cast<const _Float16*>(static_cast<const char*>(ws) + h.ws_vt_off);
  a.vt_head = h.nk_pad * d.head_dim;
  a.vt_batch = a.vt_head * d.head_count;
  a.out = static_cast<__bf16*>(out);
  a.out_batch = (int64_t)d.nq * d.head_count * d.head_dim;
  a.nq = d.nq;
  a.hc = d.head_count;
  a.batch = d.batch;
  a.c = h.c;
  a.rope = h.geom;
  a.vexp = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + h.ws_vexp_off);
  a.retry_cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + h.ws_rcnt_off);
  a.retry_rows = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + h.ws_rrows_off);
  if (d.qk_int8) {
    const char* w = static_cast<const char*>(ws);
    a.c = 1.4426950408889634f;  // log2(e): the softmax scale is inside the q codes
    a.qc = reinterpret_cast<const int8_t*>(w + h.ws_qc_off);
    a.kc = reinterpret_cast<const int8_t*>(w + h.ws_kc_off);
    a.qc_bh = h.nq_pad * d.head_dim;
    a.kc_bh = h.nk_pad * d.head_dim;
    a.qsc = reinterpret_cast<const float*>(w + h.ws_qs_off);
    a.ksc = reinterpret_cast<const float*>(w + h.ws_ks_off);
    a.nq_blocks = (int32_t)(h.nq_pad / vdit::kQuantQ);
    a.nk_blocks = (int32_t)(h.nk_pad / vdit::kQuantK);
  }
  for (int32_t b = 0; b < vdit::kMaxBatch; ++b) a.kv_len[b] = kl.len[b];
  if (vdit::launch_attn_fwd(a, d.head_dim, d.use_rope != 0, d.qk_int8 != 0, s) != hipSuccess)
    return VDIT_ERR_DEVICE;
  return VDIT_OK;
}

vdit_status_t check_out(const vdit_attn& h, const Inputs& in, void* out, const void* ws) {
  if (!out) return VDIT_ERR_INVALID_ARG;
  if (!aligned16(out)) return VDIT_ERR_ALIGNMENT;
  const size_t ob = (size_t)h.desc.batch * h.desc.nq * h.desc.head_count * h.desc.head_dim * 2;
  if (overlaps(out, ob, in.q_base, in.q_bytes) || overlaps(out, ob, in.k_base, in.k_bytes) ||
      overlaps(out, ob, in.v_base, in.v_bytes) || overlaps(out, ob, ws, h.ws_total))
    return VDIT_ERR_INVALID_ARG;
  return VDIT_OK;
}

vdit_status_t check_ws_inputs(const vdit_attn& h, const Inputs& in, const void* ws) {
  if (overlaps(ws, h.ws_total, in.q_base, in.q_bytes) || overlaps(ws, h.ws_total, in.k_base, in.k_bytes) ||
      overlaps(ws, h.ws_total, in.v_base, in.v_bytes))
    return VDIT_ERR_INVALID_ARG;
  return VDIT_OK;
}

}  // namespace

extern "C" {

vdit_status_t vdit_attn_ulysses_heads(int32_t heads_total, int32_t degree, int32_t rank, int32_t* head_begin,
                                      int32_t* head_count) {
  if (!head_begin || !head_count) return VDIT_ERR_INVALID_ARG;
  if (heads_total <= 0 || degree <= 0 || heads_total % degree != 0) return VDIT_ERR_INVALID_ARG;
  if (rank < 0 || rank >= degree) return VDIT_ERR_INVALID_ARG;
  const int32_t per = heads_total / degree;
  *head_begin = rank * per;
  *head_count = per;
  return VDIT_OK;
}

vdit_status_t vdit_attn_create(const vdit_attn_desc_t* desc, vdit_attn_t* out) {
  if (!desc || !out) return VDIT_ERR_INVALID_ARG;
  *out = nullptr;
  const vdit_status_t st = validate_desc(*desc);
  if (st != VDIT_OK) return st;

  vdit_attn* hp = new (std::nothrow) vdit_attn{};
  if (!hp) return VDIT_ERR_OUT_OF_MEMORY;
  vdit_attn& h = *hp;
  h.desc = *desc;
  if (h.desc.batch < 1) h.desc.batch = 1;
  const vdit_attn_desc_t& d = h.desc;
  const double scale = d.scale > 0.0f ? (double)d.scale : 1.0 / std::sqrt((double)d.head_dim);
  h.scale = (float)scale;
  h.c = (float)(scale * 1.4426950408889634);  // log2(e)
  h.nk_pad = ((int64_t)d.nk + vdit::kBlockN - 1) / vdit::kBlockN * vdit::kBlockN;
  h.cube = vdit::CubeGeom{};
  if (d.vsa_cubes) {
    h.cube.on = 1;
    h.cube.t = d.grid_t;
    h.cube.h = d.grid_h;
    h.cube.w = d.grid_w;
    h.cube.nct = (d.grid_t + vdit::kCube - 1) / vdit::kCube;
    h.cube.ncy = (d.grid_h + vdit::kCube - 1) / vdit::kCube;
    h.cube.ncx = (d.grid_w + vdit::kCube - 1) / vdit::kCube;
    h.cube.n = h.cube.nct * h.cube.ncy * h.cube.ncx;
  }
  h.vt_slots = h.nk_pad;
  if (d.vsa_cubes && (int64_t)h.cube.n * vdit::kBlockN > h.vt_slots) h.vt_slots = (int64_t)h.cube.n * vdit::kBlockN;
  const size_t per_head = (size_t)h.vt_slots * d.head_dim * 2;
  h.ws_vt_off = 0;
  h.ws_vt_bytes = per_head * d.head_count * d.batch;
  h.ws_kr_off = align_up(h.ws_vt_bytes, 256);
  h.ws_kr_bytes = (d.use_rope || d.vsa_cubes) ? per_head * d.head_count * d.batch : 0;
  h.ws_total = h.ws_kr_bytes ? h.ws_kr_off + h.ws_kr_bytes : h.ws_vt_bytes;
  h.nq_pad = ((int64_t)d.nq + vdit::kQuantQ - 1) / vdit::kQuantQ * vdit::kQuantQ;
  if (d.qk_int8) {
    const size_t slices = (size_t)d.head_count * d.batch;
    h.ws_qc_off = align_up(h.ws_total, 256);
    h.ws_kc_off = align_up(h.ws_qc_off + slices * h.nq_pad * d.head_dim, 256);
    h.ws_qs_off = align_up(h.ws_kc_off + slices * h.nk_pad * d.head_dim, 256);
    h.ws_ks_off = align_up(h.ws_qs_off + slices * (h.nq_pad / vdit::kQuantQ) * sizeof(float), 256);
    h.ws_total = h.ws_ks_off + slices * (h.nk_pad / vdit::kQuantK) * sizeof(float);
  }
  {
    const size_t slices = (size_t)d.head_count * d.batch;
    h.ws_vpart_off = align_up(h.ws_total, 256);
    h.ws_vexp_off = align_up(h.ws_vpart_off + slices * vdit::kVParts * sizeof(float), 256);
    h.ws_rcnt_off = align_up(h.ws_vexp_off + slices * sizeof(int32_t), 256);
    h.ws_rrows_off = align_up(h.ws_rcnt_off + slices * 2 * sizeof(int32_t), 256);
    h.ws_total = h.ws_rrows_off + slices * (size_t)d.nq * sizeof(int32_t);
  }
  h.rope_tab = nullptr;
  h.geom = vdit::RopeGeom{};

  if (hipGetDevice(&h.device) != hipSuccess) {
    delete hp;
    return VDIT_ERR_DEVICE;
  }
  if (d.use_rope) {
    std::vector<float2> tab;
    build_rope_table(d, tab, h.geom);
    if (hipMalloc(reinterpret_cast<void**>(&h.rope_tab), tab.size() * sizeof(float2)) != hipSuccess) {
      (void)hipGetLastError();
      delete hp;
      return VDIT_ERR_OUT_OF_MEMORY;
    }
    if (hipMemcpy(h.rope_tab, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(h.rope_tab);
      delete hp;
      return VDIT_ERR_DEVICE;
    }
    h.geom.tab = h.rope_tab;
  }
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    live_handles().insert(hp);
  }
  *out = hp;
  return VDIT_OK;
}

vdit_status_t vdit_attn_destroy(vdit_attn_t h) {
  if (!h) return VDIT_OK;
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    if (live_handles().erase(h) == 0) return VDIT_ERR_INVALID_ARG;
  }
  vdit_status_t st = VDIT_OK;
  if (h->rope_tab && hipFree(h->rope_tab) != hipSuccess) st = VDIT_ERR_DEVICE;
  delete h;
  return st;
}

vdit_status_t vdit_attn_workspace_bytes(vdit_attn_t h, size_t* bytes) {
  if (!is_live(h) || !bytes) return VDIT_ERR_INVALID_ARG;
  *bytes = h->ws_total;
  return VDIT_OK;
}

}  // extern "C"

namespace {

enum class Stage { kPrepare, kAttend, kBoth };

vdit_status_t run(vdit_attn_t h, const void* q, const void* k, const void* v, bool per_entry, int32_t key_len,
                  const int32_t* key_lens, void* out, void* workspace, size_t workspace_bytes, void* hip_stream,
                  Stage stage) {
  if (!is_live(h)) return VDIT_ERR_INVALID_ARG;
  Inputs in{};
  vdit_status_t st = resolve_inputs(*h, q, k, v, in);
  if (st != VDIT_OK) return st;
  if (stage != Stage::kPrepare && (st = check_out(*h, in, out, workspace)) != VDIT_OK) return st;
  KeyLens kl;
  if ((st = resolve_lens(*h, per_entry, key_len, key_lens, kl)) != VDIT_OK) return st;
  if ((st = check_call(*h, workspace, workspace_bytes)) != VDIT_OK) return st;
  if ((st = check_ws_inputs(*h, in, workspace)) != VDIT_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (stage != Stage::kAttend && (st = do_prepare(*h, in, kl, workspace, s)) != VDIT_OK) return st;
  if (stage != Stage::kPrepare) return do_attend(*h, in, kl, out, workspace, s);
  return VDIT_OK;
}

}  // namespace

// ---- internal entry points for the fixed-workspace variant (noalloc.hip)
namespace vdit {

vdit_status_t plan_workspace(vdit_attn_t h, size_t* bytes, int* device) {
  if (!is_live(h) || !bytes || !device) return VDIT_ERR_INVALID_ARG;
  *bytes = h->ws_total;
  *device = h->device;
  return VDIT_OK;
}

vdit_status_t fwd_into_workspace(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t key_len,
                                 void* out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return run(h, q, k, v, false, key_len, nullptr, out, workspace, workspace_bytes, hip_stream, Stage::kBoth);
}

}  // namespace vdit

extern "C" {

vdit_status_t vdit_attn_prepare(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t key_len,
                                void* workspace, size_t workspace_bytes, void* hip_stream) {
  return run(h, q, k, v, false, key_len, nullptr, nullptr, workspace, workspace_bytes, hip_stream, Stage::kPrepare);
}

vdit_status_t vdit_attn_attend(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t key_len,
                               void* out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return run(h, q, k, v, false, key_len, nullptr, out, workspace, workspace_bytes, hip_stream, Stage::kAttend);
}

vdit_status_t vdit_attn_fwd(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t key_len, void* out,
                            void* workspace, size_t workspace_bytes, void* hip_stream) {
  return run(h, q, k, v, false, key_len, nullptr, out, workspace, workspace_bytes, hip_stream, Stage::kBoth);
}

vdit_status_t vdit_attn_prepare_lens(vdit_attn_t h, const void* q, const void* k, const void* v,
                                     const int32_t* key_lens, void* workspace, size_t workspace_bytes,
                                     void* hip_stream) {
  return run(h, q, k, v, true, 0, key_lens, nullptr, workspace, workspace_bytes, hip_stream, Stage::kPrepare);
}

vdit_status_t vdit_attn_attend_lens(vdit_attn_t h, const void* q, const void* k, const void* v,
                                    const int32_t* key_lens, void* out, void* workspace, size_t workspace_bytes,
                                    void* hip_stream) {
  return run(h, q, k, v, true, 0, key_lens, out, workspace, workspace_bytes, hip_stream, Stage::kAttend);
}

vdit_status_t vdit_attn_fwd_lens(vdit_attn_t h, const void* q, const void* k, const void* v, const int32_t* key_lens,
                                 void* out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return run(h, q, k, v, true, 0, key_lens, out, workspace, workspace_bytes, hip_stream, Stage::kBoth);
}

static vdit_status_t pack_common(const void* src, void* dst, int32_t n, int32_t ht, int32_t d, int32_t groups,
                                 bool unpack, void* hip_stream) {
  if (!src || !dst || n <= 0 || ht <= 0 || d <= 0 || groups <= 0 || ht % groups != 0) return VDIT_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(dst) || (d * 2) % 16 != 0) return VDIT_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * ht * d * 2;
  if (overlaps(src, bytes, dst, bytes)) return VDIT_ERR_INVALID_ARG;
  if ((int64_t)ht * (d / 8) > (int64_t(1) << 30)) return VDIT_ERR_UNSUPPORTED;
  if (vdit::launch_pack(src, dst, n, ht, d, groups, unpack, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
    return VDIT_ERR_DEVICE;
  return VDIT_OK;
}

vdit_status_t vdit_pack_heads(const void* src, void* dst, int32_t n, int32_t heads_total, int32_t head_dim,
                              int32_t groups, void* hip_stream) {
  return pack_common(src, dst, n, heads_total, head_dim, groups, false, hip_stream);
}

vdit_status_t vdit_unpack_heads(const void* src, void* dst, int32_t n, int32_t heads_total, int32_t head_dim,
                                int32_t groups, void* hip_stream) {
  return pack_common(src, dst, n, heads_total, head_dim, groups, true, hip_stream);
}

vdit_status_t vdit_attn_rope_probe(vdit_attn_t h, int32_t* idx_out, void* hip_stream) {
  if (!is_live(h) || !idx_out) return VDIT_ERR_INVALID_ARG;
  if (!h->desc.use_rope) return VDIT_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return VDIT_ERR_DEVICE;
  if (vdit::launch_rope_probe(h->geom, h->desc.nq, h->desc.head_dim, idx_out, static_cast<hipStream_t>(hip_stream)) !=
      hipSuccess)
    return VDIT_ERR_DEVICE;
  return VDIT_OK;
}

}  // extern "C"

// ---- block-sparse attention over 64-token tiles
namespace {

struct VsaLayout {
  int32_t tq, tk;
  size_t tiles_off, qm_off, km_off, s_off, total;
};

int32_t tiles_of(int32_t n) { return (n + vdit::kBlockN - 1) / vdit::kBlockN; }

// query (= key) tiles of the block-sparse calls: runs of 64 tokens or cubes
int32_t vsa_q_tiles(const vdit_attn& h) { return h.cube.on ? h.cube.n : tiles_of(h.desc.nq); }
int32_t vsa_k_tiles(const vdit_attn& h) { return h.cube.on ? h.cube.n : tiles_of(h.desc.nk); }

// Workspace: the attention part (transposed v), then the kept tiles (vdit_vsa_fwd),
// the tile means of q and k and the coarse scores, each 256-byte aligned.
VsaLayout vsa_layout(const vdit_attn& h, int32_t keep) {
  const vdit_attn_desc_t& d = h.desc;
  VsaLayout l{};
  l.tq = vsa_q_tiles(h);
  l.tk = vsa_k_tiles(h);
  const size_t bh = (size_t)d.batch * d.head_count;
  l.tiles_off = align_up(h.ws_total, 256);
  l.qm_off = align_up(l.tiles_off + bh * l.tq * (size_t)keep * sizeof(int32_t), 256);
  l.km_off = align_up(l.qm_off + bh * l.tq * (size_t)d.head_dim * sizeof(float), 256);
  l.s_off = align_up(l.km_off + bh * l.tk * (size_t)d.head_dim * sizeof(float), 256);
  l.total = l.s_off + bh * l.tq * (size_t)l.tk * sizeof(float);
  return l;
}

vdit_status_t vsa_check(const vdit_attn* h, int32_t keep) {
  if (!is_live(h)) return VDIT_ERR_INVALID_ARG;
  const vdit_attn_desc_t& d = h->desc;
  if (d.use_key_mask || d.use_rope || d.qk_int8) return VDIT_ERR_UNSUPPORTED;
  const int32_t tk = vsa_k_tiles(*h);
  if (tk > vdit::kVsaMaxTiles) return VDIT_ERR_UNSUPPORTED;
  if (keep < 1 || keep > tk) return VDIT_ERR_INVALID_ARG;
  if (keep > vdit::kVsaMaxKeep) return VDIT_ERR_UNSUPPORTED;
  return VDIT_OK;
}

vdit_status_t vsa_call_checks(const vdit_attn& h, const VsaLayout& l, void* ws, size_t ws_bytes) {
  if (!ws || ws_bytes < l.total) return VDIT_ERR_WORKSPACE;
  if (!aligned16(ws)) return VDIT_ERR_ALIGNMENT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h.device) return VDIT_ERR_DEVICE;
  return VDIT_OK;
}

bool ws_overlaps_inputs(const Inputs& in, const void* p, size_t n) {
  return overlaps(p, n, in.q_base, in.q_bytes) || overlaps(p, n, in.k_base, in.k_bytes) ||
         overlaps(p, n, in.v_base, in.v_bytes);
}

vdit_status_t do_vsa_select(const vdit_attn& h, const Inputs& in, const VsaLayout& l, int32_t keep,
                            int32_t* tiles, void* ws, hipStream_t s) {
  const vdit_attn_desc_t& d = h.desc;
  char* w = static_cast<char*>(ws);
  const int32_t bh = d.batch * d.head_count;
  vdit::VsaMeanArgs m{};
  m.hc = d.head_count;
  m.bh = bh;
  m.x = in.q;
  m.row = in.q_row;
  m.batch = in.q_batch;
  m.mean = reinterpret_cast<float*>(w + l.qm_off);
  m.n = d.nq;
  m.tiles = l.tq;
  m.cube = h.cube;
  if (vdit::launch_vsa_means(m, d.head_dim, s) != hipSuccess) return VDIT_ERR_DEVICE;
  m.x = in.k;
  m.row = in.kv_row;
  m.batch = in.kv_batch;
  m.mean = reinterpret_cast<float*>(w + l.km_off);
  m.n = d.nk;
  m.tiles = l.tk;
  if (vdit::launch_vsa_means(m, d.head_dim, s) != hipSuccess) return VDIT_ERR_DEVICE;
  vdit::VsaSelectArgs a{};
  a.qm = reinterpret_cast<const float*>(w + l.qm_off);
  a.km = reinterpret_cast<const float*>(w + l.km_off);
  a.s = reinterpret_cast<float*>(w + l.s_off);
  a.tiles = tiles;
  a.tq = l.tq;
  a.tk = l.tk;
  a.keep = keep;
  a.d = d.head_dim;
  a.bh = bh;
  if (vdit::launch_vsa_select(a, s) != hipSuccess) return VDIT_ERR_DEVICE;
  return VDIT_OK;
}

vdit_status_t do_vsa_attend(const vdit_attn& h, const Inputs& in, int32_t keep, const int32_t* tiles, void* out,
                            void* ws, hipStream_t s) {
  const vdit_attn_desc_t& d = h.desc;
  KeyLens kl;
  vdit_status_t st = resolve_lens(h, false, 0, nullptr, kl);
  if (st != VDIT_OK) return st;
  const bool cubes = h.cube.on != 0;
  if ((st = do_prepare(h, in, kl, ws, s, cubes)) != VDIT_OK) return st;
  vdit::AttnArgs a{};
  a.q = in.q;
  a.q_row = in.q_row;
  a.q_head = d.head_dim;
  a.q_batch = in.q_batch;
  if (cubes) {
    // k in cube order from the workspace, every cube one 64-slot key tile
    a.k = reinterpret_cast<const __bf16*>(static_cast<const char*>(ws) + h.ws_kr_off);
    a.k_row = d.head_dim;
    a.k_head = h.vt_slots * d.head_dim;
    a.k_batch = a.k_head * d.head_count;
    a.cube = h.cube;
  } else {
    a.k = in.k;
    a.k_row = in.kv_row;
    a.k_head = d.head_dim;
    a.k_batch = in.kv_batch;
  }
  a.vt = reinterpret_cast<const _Float16*>(static_cast<const char*>(ws) + h.ws_vt_off);
  a.vt_head = (cubes ? h.vt_slots : h.nk_pad) * d.head_dim;
  a.vt_batch = a.vt_head * d.head_count;
  a.out = static_cast<__bf16*>(out);
  a.out_batch = (int64_t)d.nq * d.head_count * d.head_dim;
  a.nq = d.nq;
  a.hc = d.head_count;
  a.batch = d.batch;
  a.c = h.c;
  a.tiles = tiles;
  a.keep = keep;
  a.vexp = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + h.ws_vexp_off);
  for (int32_t b = 0; b < vdit::kMaxBatch; ++b)
    a.kv_len[b] = cubes && b < d.batch ? (int32_t)(h.cube.n * vdit::kBlockN) : kl.len[b];
  if (vdit::launch_attn_sparse(a, d.head_dim, s) != hipSuccess) return VDIT_ERR_DEVICE;
  return VDIT_OK;
}

}  // namespace

extern "C" {

vdit_status_t vdit_vsa_keep(vdit_attn_t h, double sparsity, int32_t* keep) {
  if (!is_live(h) || !keep) return VDIT_ERR_INVALID_ARG;
  if (!(sparsity >= 0.0 && sparsity < 1.0)) return VDIT_ERR_INVALID_ARG;
  const int32_t tk = vsa_k_tiles(*h);
  const double want = std::ceil((1.0 - sparsity) * (double)tk);
  *keep = want < 1.0 ? 1 : (want > (double)tk ? tk : (int32_t)want);
  return VDIT_OK;
}

vdit_status_t vdit_vsa_workspace_bytes(vdit_attn_t h, int32_t keep, size_t* bytes) {
  if (!bytes) return VDIT_ERR_INVALID_ARG;
  const vdit_status_t st = vsa_check(h, keep);
  if (st != VDIT_OK) return st;
  *bytes = vsa_layout(*h, keep).total;
  return VDIT_OK;
}

vdit_status_t vdit_vsa_select(vdit_attn_t h, const void* q, const void* k, int32_t keep, int32_t* tiles,
                              void* workspace, size_t workspace_bytes, void* hip_stream) {
  vdit_status_t st = vsa_check(h, keep);
  if (st != VDIT_OK) return st;
  Inputs in{};
  // the packed layout carries k inside q; with separate tensors v is not read
  const void* v = h->desc.layout == VDIT_LAYOUT_N3HD ? nullptr : k;
  if ((st = resolve_inputs(*h, q, k, v, in)) != VDIT_OK) return st;
  if (!tiles) return VDIT_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(tiles) & 3u) return VDIT_ERR_ALIGNMENT;
  const VsaLayout l = vsa_layout(*h, keep);
  if ((st = vsa_call_checks(*h, l, workspace, workspace_bytes)) != VDIT_OK) return st;
  const size_t tb = (size_t)h->desc.batch * h->desc.head_count * l.tq * keep * sizeof(int32_t);
  if (ws_overlaps_inputs(in, workspace, l.total) || ws_overlaps_inputs(in, tiles, tb) ||
      overlaps(tiles, tb, workspace, l.total))
    return VDIT_ERR_INVALID_ARG;
  return do_vsa_select(*h, in, l, keep, tiles, workspace, static_cast<hipStream_t>(hip_stream));
}

vdit_status_t vdit_vsa_attend(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t keep,
                              const int32_t* tiles, void* out, void* workspace, size_t workspace_bytes,
                              void* hip_stream) {
  vdit_status_t st = vsa_check(h, keep);
  if (st != VDIT_OK) return st;
  Inputs in{};
  if ((st = resolve_inputs(*h, q, k, v, in)) != VDIT_OK) return st;
  if ((st = check_out(*h, in, out, workspace)) != VDIT_OK) return st;
  if (!tiles) return VDIT_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(tiles) & 3u) return VDIT_ERR_ALIGNMENT;
  // the attention part of the workspace is all this call writes besides out
  if (!workspace || workspace_bytes < h->ws_total) return VDIT_ERR_WORKSPACE;
  if (!aligned16(workspace)) return VDIT_ERR_ALIGNMENT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return VDIT_ERR_DEVICE;
  const size_t tb = (size_t)h->desc.batch * h->desc.head_count * vsa_q_tiles(*h) * keep * sizeof(int32_t);
  const size_t ob = (size_t)h->desc.batch * h->desc.nq * h->desc.head_count * h->desc.head_dim * 2;
  if (ws_overlaps_inputs(in, workspace, h->ws_total) || overlaps(tiles, tb, workspace, h->ws_total) ||
      overlaps(tiles, tb, out, ob))
    return VDIT_ERR_INVALID_ARG;
  return do_vsa_attend(*h, in, keep, tiles, out, workspace, static_cast<hipStream_t>(hip_stream));
}

vdit_status_t vdit_vsa_fwd(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t keep, void* out,
                           void* workspace, size_t workspace_bytes, void* hip_stream) {
  vdit_status_t st = vsa_check(h, keep);
  if (st != VDIT_OK) return st;
  Inputs in{};
  if ((st = resolve_inputs(*h, q, k, v, in)) != VDIT_OK) return st;
  const VsaLayout l = vsa_layout(*h, keep);
  if ((st = vsa_call_checks(*h, l, workspace, workspace_bytes)) != VDIT_OK) return st;
  const size_t ob = (size_t)h->desc.batch * h->desc.nq * h->desc.head_count * h->desc.head_dim * 2;
  if (!out) return VDIT_ERR_INVALID_ARG;
  if (!aligned16(out)) return VDIT_ERR_ALIGNMENT;
  if (ws_overlaps_inputs(in, workspace, l.total) || ws_overlaps_inputs(in, out, ob) ||
      overlaps(out, ob, workspace, l.total))
    return VDIT_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  int32_t* tiles = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + l.tiles_off);
  if ((st = do_vsa_select(*h, in, l, keep, tiles, workspace, s)) != VDIT_OK) return st;
  return do_vsa_attend(*h, in, keep, tiles, out, workspace, s);
}

const char* vdit_status_string(vdit_status_t s) {
  switch (s) {
    case VDIT_OK: return "VDIT_OK";
    case VDIT_ERR_INVALID_ARG: return "VDIT_ERR_INVALID_ARG: invalid argument or shape";
    case VDIT_ERR_UNSUPPORTED: return "VDIT_ERR_UNSUPPORTED: valid request outside what the kernels implement";
    case VDIT_ERR_ALIGNMENT: return "VDIT_ERR_ALIGNMENT: device pointer not 16-byte aligned";
    case VDIT_ERR_OUT_OF_MEMORY: return "VDIT_ERR_OUT_OF_MEMORY: device table allocation failed";
    case VDIT_ERR_DEVICE: return "VDIT_ERR_DEVICE: HIP call or kernel launch failed, or wrong device current";
    case VDIT_ERR_WORKSPACE: return "VDIT_ERR_WORKSPACE: workspace missing or too small";
  }
  return "VDIT_ERR_UNKNOWN: unknown status code";
}

}  // extern "C"

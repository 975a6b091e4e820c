// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; no GPU is touched): every path here
// returns a status before any kernel launch. Exits non-zero on the first wrong
// status; a sanitizer finding aborts the run.
#include <cstdio>
#include <cstring>

#include "vdit_attn.h"

static int failures = 0;

static void expect(const char* what, vdit_status_t got, vdit_status_t want) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, (int)got, (int)want);
    ++failures;
  }
}

static vdit_attn_desc_t good() {
  vdit_attn_desc_t d;
  std::memset(&d, 0, sizeof(d));
  d.nq = 300;
  d.nk = 300;
  d.heads_total = 4;
  d.head_dim = 128;
  d.layout = VDIT_LAYOUT_NHD;
  d.head_begin = 1;
  d.head_count = 2;
  d.batch = 1;
  return d;
}

int main() {
  int32_t b = -1, c = -1;
  expect("ulysses 40/4/3", vdit_attn_ulysses_heads(40, 4, 3, &b, &c), VDIT_OK);
  if (b != 30 || c != 10) {
    std::printf("FAIL ulysses share %d %d\n", b, c);
    ++failures;
  }
  expect("ulysses 40/3", vdit_attn_ulysses_heads(40, 3, 0, &b, &c), VDIT_ERR_INVALID_ARG);
  expect("ulysses rank", vdit_attn_ulysses_heads(40, 4, 4, &b, &c), VDIT_ERR_INVALID_ARG);
  expect("ulysses null", vdit_attn_ulysses_heads(40, 4, 0, nullptr, &c), VDIT_ERR_INVALID_ARG);

  vdit_attn_t h = nullptr;
  struct Bad {
    const char* what;
    void (*edit)(vdit_attn_desc_t&);
    vdit_status_t want;
  };
  const Bad bads[] = {
      {"head_dim 96", [](vdit_attn_desc_t& d) { d.head_dim = 96; }, VDIT_ERR_UNSUPPORTED},
      {"nq 0", [](vdit_attn_desc_t& d) { d.nq = 0; }, VDIT_ERR_INVALID_ARG},
      {"layout 7", [](vdit_attn_desc_t& d) { d.layout = 7; }, VDIT_ERR_INVALID_ARG},
      {"packed nq != nk", [](vdit_attn_desc_t& d) { d.layout = VDIT_LAYOUT_N3HD; d.nk = 299; }, VDIT_ERR_INVALID_ARG},
      {"head range", [](vdit_attn_desc_t& d) { d.head_begin = 3; }, VDIT_ERR_INVALID_ARG},
      {"batch 65", [](vdit_attn_desc_t& d) { d.batch = 65; }, VDIT_ERR_UNSUPPORTED},
      {"batch -1", [](vdit_attn_desc_t& d) { d.batch = -1; }, VDIT_ERR_INVALID_ARG},
      {"nan scale", [](vdit_attn_desc_t& d) { d.scale = __builtin_nanf(""); }, VDIT_ERR_INVALID_ARG},
      {"mask flag 2", [](vdit_attn_desc_t& d) { d.use_key_mask = 2; }, VDIT_ERR_INVALID_ARG},
      {"int8 with d 64", [](vdit_attn_desc_t& d) { d.qk_int8 = 1; d.head_dim = 64; }, VDIT_ERR_UNSUPPORTED},
      {"rope grid", [](vdit_attn_desc_t& d) {
         d.use_rope = 1; d.grid_t = 3; d.grid_h = 10; d.grid_w = 11;
         d.rope_dim_t = 44; d.rope_dim_h = 42; d.rope_dim_w = 42; d.rope_base = 10000.0; }, VDIT_ERR_INVALID_ARG},
      {"rope odd band", [](vdit_attn_desc_t& d) {
         d.use_rope = 1; d.grid_t = 3; d.grid_h = 10; d.grid_w = 10;
         d.rope_dim_t = 43; d.rope_dim_h = 43; d.rope_dim_w = 42; d.rope_base = 10000.0; }, VDIT_ERR_INVALID_ARG},
      {"rope base 0", [](vdit_attn_desc_t& d) {
         d.use_rope = 1; d.grid_t = 3; d.grid_h = 10; d.grid_w = 10;
         d.rope_dim_t = 44; d.rope_dim_h = 42; d.rope_dim_w = 42; d.rope_base = 0.0; }, VDIT_ERR_INVALID_ARG},
      {"cube grid", [](vdit_attn_desc_t& d) { d.vsa_cubes = 1; d.grid_t = 3; d.grid_h = 10; d.grid_w = 11; },
       VDIT_ERR_INVALID_ARG},
      {"cube flag 2", [](vdit_attn_desc_t& d) { d.vsa_cubes = 2; d.grid_t = 3; d.grid_h = 10; d.grid_w = 10; },
       VDIT_ERR_INVALID_ARG},
      {"cube count", [](vdit_attn_desc_t& d) {
         d.nq = d.nk = 532480; d.vsa_cubes = 1; d.grid_t = 8; d.grid_h = 256; d.grid_w = 260; }, VDIT_ERR_UNSUPPORTED},
  };
  for (const Bad& x : bads) {
    vdit_attn_desc_t d = good();
    x.edit(d);
    expect(x.what, vdit_attn_create(&d, &h), x.want);
    if (h != nullptr) {
      std::printf("FAIL %s: handle set on error\n", x.what);
      ++failures;
    }
  }
  expect("create null desc", vdit_attn_create(nullptr, &h), VDIT_ERR_INVALID_ARG);
  vdit_attn_desc_t d = good();
  expect("create null out", vdit_attn_create(&d, nullptr), VDIT_ERR_INVALID_ARG);

  // handles never created: rejected without being dereferenced
  char fake_storage[64];
  vdit_attn_t bogus = reinterpret_cast<vdit_attn_t>(fake_storage);
  size_t n = 0;
  int32_t k = 0;
  expect("destroy null", vdit_attn_destroy(nullptr), VDIT_OK);
  expect("destroy bogus", vdit_attn_destroy(bogus), VDIT_ERR_INVALID_ARG);
  expect("workspace bogus", vdit_attn_workspace_bytes(bogus, &n), VDIT_ERR_INVALID_ARG);
  expect("fwd bogus", vdit_attn_fwd(bogus, nullptr, nullptr, nullptr, 1, nullptr, nullptr, 0, nullptr),
         VDIT_ERR_INVALID_ARG);
  const int32_t lens[2] = {5, 7};
  expect("fwd_lens bogus", vdit_attn_fwd_lens(bogus, nullptr, nullptr, nullptr, lens, nullptr, nullptr, 0, nullptr),
         VDIT_ERR_INVALID_ARG);
  expect("rope probe bogus", vdit_attn_rope_probe(bogus, nullptr, nullptr), VDIT_ERR_INVALID_ARG);
  expect("vsa keep bogus", vdit_vsa_keep(bogus, 0.8, &k), VDIT_ERR_INVALID_ARG);
  expect("vsa ws bogus", vdit_vsa_workspace_bytes(bogus, 3, &n), VDIT_ERR_INVALID_ARG);
  expect("vsa select bogus", vdit_vsa_select(bogus, nullptr, nullptr, 3, nullptr, nullptr, 0, nullptr),
         VDIT_ERR_INVALID_ARG);
  expect("vsa fwd bogus", vdit_vsa_fwd(bogus, nullptr, nullptr, nullptr, 3, nullptr, nullptr, 0, nullptr),
         VDIT_ERR_INVALID_ARG);

  // pack validation (pointers are never dereferenced on these paths)
  void* p = reinterpret_cast<void*>(0x10000);
  void* q = reinterpret_cast<void*>(0x20000000);
  expect("pack null", vdit_pack_heads(nullptr, q, 10, 40, 128, 4, nullptr), VDIT_ERR_INVALID_ARG);
  expect("pack groups", vdit_pack_heads(p, q, 10, 40, 128, 3, nullptr), VDIT_ERR_INVALID_ARG);
  expect("pack misaligned", vdit_unpack_heads(p, reinterpret_cast<void*>(0x20000008), 10, 40, 128, 4, nullptr),
         VDIT_ERR_ALIGNMENT);
  expect("pack overlap", vdit_pack_heads(p, reinterpret_cast<void*>(0x10000 + 64), 10, 40, 128, 4, nullptr),
         VDIT_ERR_INVALID_ARG);

  for (int s = 0; s <= 7; ++s) {
    const char* str = vdit_status_string(static_cast<vdit_status_t>(s));
    if (!str || !*str) {
      std::printf("FAIL status string %d\n", s);
      ++failures;
    }
  }
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}

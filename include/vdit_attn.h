/*
 * vdit_attn — non-causal multi-head attention for video diffusion transformers
 * on AMD Instinct MI355X (gfx950), one device's share of the heads.
 *
 * The operation. In a video DiT split across devices with Ulysses sequence
 * parallelism, an all-to-all before every attention layer hands each device
 * the whole spatio-temporal token sequence for a slice of the heads (fal.ai,
 * "Generate video with WAN 2.2 across four GPUs", section "Splitting one
 * generation across four GPUs": four GPUs each attend over the full sequence
 * for 10 of the 40 heads). The attention itself is non-causal and may take a
 * key mask (ComfyUI issue "MultiGPU Work Units": the WAN forward pass calls
 * sageattn with attn_mask and is_causal=False). This library computes, for
 * every selected head h and query token i,
 *
 *     out[i, h - head_begin, :] = sum_j w_ij v[j, h, :],
 *     w_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij),
 *     s_ij = scale * <q'[i, h, :], k'[j, h, :]>,   j < key_len,
 *
 * where q' and k' are q and k, optionally rotated by a 3D rotary position
 * embedding over a (T, H, W) latent grid (below). Sequence parallelism is
 * numerically faithful to a single device (LTX-2 "Multi-GPU Inference",
 * section "Capabilities"); here a head share computes bit-for-bit the same
 * values as the same heads inside an all-heads call.
 *
 * 3D RoPE reading (the pages name no formula): token n of the grid, w fastest,
 * sits at t = n / (H*W), y = (n / W) % H, x = n % W. The head dimension is cut
 * into three consecutive bands of widths (rope_dim_t, rope_dim_h, rope_dim_w);
 * band b rotates its adjacent pairs (2i, 2i+1) by theta = pos_b * base^(-2i/D_b).
 * cos/sin are tabulated on the host in double precision and rounded to float;
 * the rotation runs in float (a*c - b*s, a*s + b*c, each as one fused
 * multiply-add) and the result is rounded to bfloat16 before the products.
 *
 * Numerics: q.k products in bfloat16 with float32 accumulation; softmax in
 * float32, taken relative to a fixed per-row reference (the maximum over the
 * first 64 keys; rows where a weight would leave the float16 range are listed and
 * recomputed with the exact maximum by a second launch); the weights are rounded to float16 and
 * v is converted once to float16 for the weighted sum (float32 accumulation),
 * after scaling each (entry, head) of v by the power of two 2^e that brings its
 * largest |v| over the valid keys into [2^14, 2^15) (e in [-113, 160]); the
 * output is multiplied by 2^-e, which undoes the scaling exactly. So every
 * finite bfloat16 v works: none overflows, and values down to 2^-29 of the
 * head's largest convert to float16 exactly. The output is rounded to bfloat16
 * (nearest even).
 * Batch. One call may carry B independent sequences of the same shape, e.g.
 * the positive and negative conditioning of classifier-free guidance (ComfyUI
 * issue "MultiGPU Work Units": diffusion models usually run two conditionings,
 * positive and negative; the fal.ai page, section "Defining the request
 * schema", exposes the guidance scales). Every tensor then gains a leading [B]
 * dimension and each entry is computed exactly as a call with B = 1 would.
 *
 * Conventions for every entry point:
 *   - all tensors live in device memory owned by the caller; the library
 *     never frees or keeps them past the call;
 *   - pointers passed to compute calls must be 16-byte aligned;
 *   - calls taking `hip_stream` (a hipStream_t; NULL = default stream) only
 *     enqueue kernels on that stream: they never allocate, fill memory with the
 *     runtime or synchronise the host, so they may be captured in a HIP graph
 *     (scalar arguments such as key_len are then fixed at capture);
 *   - errors come back as vdit_status_t values, never as exceptions or aborts;
 *     a shape or argument error is reported before anything is enqueued;
 *   - the handle is immutable after create: calls on one handle may run on
 *     different streams concurrently if their workspaces are distinct;
 *   - compute calls must run with the device current that was current at create.
 */
#ifndef VDIT_ATTN_H
#define VDIT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct vdit_attn* vdit_attn_t;

typedef enum {
  VDIT_OK = 0,
  VDIT_ERR_INVALID_ARG = 1,    /* NULL pointer, bad shape, bad head range, bad key_len, aliasing */
  VDIT_ERR_UNSUPPORTED = 2,    /* valid request outside what the kernels implement (e.g. d not 64/128) */
  VDIT_ERR_ALIGNMENT = 3,      /* a device pointer is not 16-byte aligned */
  VDIT_ERR_OUT_OF_MEMORY = 4,  /* the small create-time device tables could not be allocated */
  VDIT_ERR_DEVICE = 5,         /* a HIP call or kernel launch failed, or the wrong device is current */
  VDIT_ERR_WORKSPACE = 6       /* workspace NULL or smaller than vdit_attn_workspace_bytes() */
} vdit_status_t;

typedef enum {
  VDIT_LAYOUT_NHD = 0,  /* q [nq, Ht, d], k and v [nk, Ht, d]; bfloat16, contiguous */
  VDIT_LAYOUT_N3HD = 1  /* one packed tensor [n, 3, Ht, d] bfloat16 (index 0 = q, 1 = k, 2 = v); nq == nk */
} vdit_layout_t;

/*
 * Problem description, fixed at create. Sizes in elements.
 *   nq, nk          query and key tokens (self-attention: equal; text cross-attention:
 *                   nk = text length)
 *   heads_total     Ht, heads present in the tensors (e.g. 40)
 *   head_dim        d, 64 or 128
 *   layout          vdit_layout_t
 *   head_begin/count  selected heads [head_begin, head_begin + head_count) of Ht; the
 *                   output holds only these, in order
 *   scale           softmax scale; <= 0 selects 1/sqrt(d); NaN or inf is rejected
 *   use_key_mask    0: all nk keys; 1: only keys j < key_len (key_len given per call)
 *   use_rope        1: rotate q and k by the 3D RoPE above (requires nq == nk)
 *   grid_t/h/w      latent grid, grid_t * grid_h * grid_w == nq, token n at
 *                   t = n / (grid_h grid_w), y = (n / grid_w) % grid_h, x = n % grid_w
 *                   (used iff use_rope or vsa_cubes)
 *   rope_dim_t/h/w  band widths, each even and > 0, summing to d (used iff use_rope)
 *   rope_base       base of the frequencies, > 0 and finite (used iff use_rope)
 *   batch           B, sequences per call (0 is read as 1; at most 64, and B * head_count
 *                   at most 65535, else UNSUPPORTED). Shapes below then read
 *                   q [B, nq, Ht, d], k and v [B, nk, Ht, d], packed [B, n, 3, Ht, d],
 *                   out [B, nq, head_count, d].
 *   qk_int8         1: q.k on int8 codes, quantized per block by prepare (the per-block
 *                   int8 step that the WAN forward pass runs through SageAttention,
 *                   ComfyUI issue "MultiGPU Work Units": per_block_int8(q, k, sm_scale)).
 *                   Reading: symmetric codes, one scale per block of 128 query / 64 key
 *                   tokens of one (entry, head), q multiplied by the softmax scale first;
 *                   scale = amax / 127 (float32, IEEE division; 1 if below 2^-100),
 *                   code = round-half-even(x / scale) clamped to [-127, 127]; scores =
 *                   q scale * k scale * integer dot product. Softmax and the weighted sum
 *                   are as without it. Needs d = 128, no RoPE and nk <= 262144
 *                   (UNSUPPORTED otherwise). Workspace with qk_int8, after the regions
 *                   below, each region starting at the next multiple of 256 bytes:
 *                   q codes int8 [B * head_count][ceil(nq/128)*128][d], k codes int8
 *                   [B * head_count][ceil(nk/64)*64][d], q scales float
 *                   [B * head_count][ceil(nq/128)], k scales float [B * head_count][ceil(nk/64)].
 *   vsa_cubes       1: the block-sparse calls (vdit_vsa_*) tile q and k as 4 x 4 x 4
 *                   cubes of the latent grid instead of runs of 64 tokens (see there);
 *                   needs nq == nk == grid_t * grid_h * grid_w and at most 8192 cubes
 *                   (UNSUPPORTED beyond). The dense calls ignore it.
 */
typedef struct {
  int32_t nq;
  int32_t nk;
  int32_t heads_total;
  int32_t head_dim;
  int32_t layout;
  int32_t head_begin;
  int32_t head_count;
  float scale;
  int32_t use_key_mask;
  int32_t use_rope;
  int32_t grid_t, grid_h, grid_w;
  int32_t rope_dim_t, rope_dim_h, rope_dim_w;
  double rope_base;
  int32_t batch;
  int32_t qk_int8;
  int32_t vsa_cubes;
} vdit_attn_desc_t;

/*
 * Head share of one rank under Ulysses sequence parallelism of `degree` ranks:
 * heads [rank * Ht / degree, (rank + 1) * Ht / degree). fal.ai "Generate video
 * with WAN 2.2 across four GPUs", sections "Splitting one generation across
 * four GPUs" (10 of 40 heads per GPU at degree 4) and "Tuning cost and GPU
 * count" (the degree must divide the head count; FastVideo "Pair two NVIDIA DGX
 * Sparks", section "What we are not claiming", states the same for sp_size).
 * Host only. INVALID_ARG if degree <= 0, heads_total <= 0, heads_total % degree
 * != 0, rank outside [0, degree), or an output pointer is NULL.
 */
vdit_status_t vdit_attn_ulysses_heads(int32_t heads_total, int32_t degree, int32_t rank,
                                      int32_t* head_begin, int32_t* head_count);

/*
 * Validate `desc` and build a plan: tile shapes and launch grid are fixed here
 * for the shape, with no tuning at run time (the fal.ai page, section "Converting
 * once, starting the runner, warming up", notes that per-shape autotuning costs
 * a cold request tens of seconds). With use_rope, the cos/sin tables are built in
 * double precision, rounded to float and copied to the current device (the only
 * device memory the handle owns). Shape errors return INVALID_ARG or UNSUPPORTED
 * without touching the device. On success *out receives a handle that the caller
 * releases with vdit_attn_destroy.
 */
vdit_status_t vdit_attn_create(const vdit_attn_desc_t* desc, vdit_attn_t* out);

/* Release a handle and its tables. NULL is accepted (VDIT_OK). */
vdit_status_t vdit_attn_destroy(vdit_attn_t h);

/*
 * Bytes of caller-provided device workspace that prepare/attend/fwd need for the
 * largest key length of this plan: v transposed to float16 per entry and head
 * ([B][head_count][ceil(nk/64)*64][d], 2 bytes) and, with use_rope, the rotated keys
 * (same shape, bfloat16); with vsa_cubes both regions are present and sized for
 * max(ceil(nk/64), cubes) 64-key tiles per entry and head (the block-sparse calls
 * lay them out [B][head_count][cubes * 64][d], v transposed and k in cube order);
 * then the qk_int8 regions (above), then the range of v:
 * float [B][head_count][64] partial maxima of |v| and int32 [B][head_count] scaling
 * exponents e; then the retry list of the rows whose float16 weights overflowed:
 * int32 [B][head_count][2] counters (cleared by prepare, zero again after attend)
 * and int32 [B][head_count][nq] rows. Each region after the first starts at the
 * next multiple of 256 bytes. Host only.
 */
vdit_status_t vdit_attn_workspace_bytes(vdit_attn_t h, size_t* bytes);

/*
 * The whole forward pass on `hip_stream`: vdit_attn_prepare then vdit_attn_attend.
 *   q, k, v    NHD: q [nq, Ht, d], k and v [nk, Ht, d] (bfloat16).
 *              N3HD: q is the packed [n, 3, Ht, d] tensor; k and v must be NULL.
 *   key_len    used iff use_key_mask: 1 <= key_len <= nk (keys j >= key_len are
 *              excluded; their k and v contents are never read); otherwise ignored.
 *              With B > 1 it applies to every entry (see the _lens calls below).
 *   out        bfloat16 [nq, head_count, d], contiguous; must not overlap the inputs
 *              or the workspace.
 *   workspace  >= vdit_attn_workspace_bytes() bytes of device memory; its contents
 *              are overwritten.
 */
vdit_status_t vdit_attn_fwd(vdit_attn_t h, const void* q, const void* k, const void* v,
                            int32_t key_len, void* out, void* workspace, size_t workspace_bytes,
                            void* hip_stream);

/*
 * First stage of fwd: finds the range of v (heads of the share, keys < key_len)
 * and writes v, scaled by 2^e, transposed and converted to float16 into the
 * workspace, zero-filled up to the next multiple of 64 keys; with use_rope also the rotated keys (bfloat16); with
 * qk_int8 the int8 codes and scales of q and of the valid keys. Arguments
 * as for fwd (q is read only for the N3HD layout, where it is the packed tensor).
 */
vdit_status_t vdit_attn_prepare(vdit_attn_t h, const void* q, const void* k, const void* v,
                                int32_t key_len, void* workspace, size_t workspace_bytes,
                                void* hip_stream);

/*
 * Second stage of fwd: the attention kernel proper. Reads q (and, without
 * RoPE, k) from the inputs and the prepared workspace from vdit_attn_prepare,
 * which must have been enqueued before it with the same inputs and key_len.
 * Arguments as for fwd.
 */
vdit_status_t vdit_attn_attend(vdit_attn_t h, const void* q, const void* k, const void* v,
                               int32_t key_len, void* out, void* workspace, size_t workspace_bytes,
                               void* hip_stream);

/*
 * vdit_attn_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The workspace regions (vdit_attn_workspace_bytes)
 * live instead in a fixed 256 MiB device array of the library, one copy per GPU,
 * reserved while the library is loaded and looked up on the first call on each
 * device. The call allocates nothing. UNSUPPORTED if the plan needs more than
 * 256 MiB of workspace (one head share of 10 heads at 75600 tokens needs
 * 194 MB and fits). Every call on a GPU uses that GPU's one array: calls that overlap in
 * time on one GPU (other streams, other threads) race and give undefined
 * results; calls ordered on one stream are safe. Nothing from an earlier call is
 * read. Other arguments and errors as for vdit_attn_fwd.
 */
vdit_status_t vdit_attn_fwd_noalloc(vdit_attn_t h, const void* q, const void* k, const void* v,
                                    int32_t key_len, void* out, void* hip_stream);

/*
 * fwd, prepare and attend with one key length per batch entry, for batches whose
 * sequences mask different numbers of keys (e.g. positive and negative prompts of
 * different text lengths under classifier-free guidance). key_lens: host array of
 * B int32 values, read during the call only; used iff use_key_mask, then each must
 * satisfy 1 <= key_lens[b] <= nk and the pointer must not be NULL (INVALID_ARG
 * otherwise); NULL is accepted without use_key_mask. prepare and attend must see
 * the same lengths. Other arguments as for fwd / prepare / attend.
 */
vdit_status_t vdit_attn_fwd_lens(vdit_attn_t h, const void* q, const void* k, const void* v,
                                 const int32_t* key_lens, void* out, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);
vdit_status_t vdit_attn_prepare_lens(vdit_attn_t h, const void* q, const void* k, const void* v,
                                     const int32_t* key_lens, void* workspace, size_t workspace_bytes,
                                     void* hip_stream);
vdit_status_t vdit_attn_attend_lens(vdit_attn_t h, const void* q, const void* k, const void* v,
                                    const int32_t* key_lens, void* out, void* workspace,
                                    size_t workspace_bytes, void* hip_stream);

/*
 * Layout change for the Ulysses exchange (fal.ai page, section "Splitting one
 * generation across four GPUs": tokens are traded for heads at every attention
 * layer; LTX-2 "Multi-GPU Inference", section "Requirements", names a dedicated
 * all-to-all kernel for it). pack: src [n, Ht, d] -> dst [groups, n, Ht/groups, d],
 * i.e. dst[g, t, j, :] = src[t, g * Ht/groups + j, :]. unpack is the inverse.
 * Pure 2-byte-element permutation (bit-exact). INVALID_ARG if groups does not
 * divide Ht, a size is <= 0, a pointer is NULL or the buffers overlap; ALIGNMENT
 * if a pointer is not 16-byte aligned or d * 2 is not a multiple of 16.
 */
vdit_status_t vdit_pack_heads(const void* src, void* dst, int32_t n, int32_t heads_total,
                              int32_t head_dim, int32_t groups, void* hip_stream);
vdit_status_t vdit_unpack_heads(const void* src, void* dst, int32_t n, int32_t heads_total,
                                int32_t head_dim, int32_t groups, void* hip_stream);

/*
 * Debug probe of the RoPE index mapping the kernels use: for every query token n
 * in [0, nq) and pair p in [0, d/2), writes five int32 values
 * idx_out[(n * d/2 + p) * 5 + {0..4}] = (t, y, x, band, i), computed by the same
 * device code that rotates q and k. idx_out: device memory, nq * d/2 * 5 int32.
 * INVALID_ARG if the handle was created without use_rope or idx_out is NULL.
 */
vdit_status_t vdit_attn_rope_probe(vdit_attn_t h, int32_t* idx_out, void* hip_stream);

/*
 * Block-sparse attention over 64-token tiles (video sparse attention). FastVideo
 * "Pair two NVIDIA DGX Sparks": section "3. Generate one FastH3 clip on both
 * GPUs" names the VSA attention kernels, and section "Released V2, FastH3-QAD-v2
 * and Trim NVFP4 stacks" runs them at sparsity 0.8 with 64-token tiles. Nothing
 * more is stated; the reading implemented (that of the published video sparse
 * attention method, without its learned gates and coarse output branch) is:
 *
 *   tiles      runs of 64 consecutive tokens as the tensors hold them (the last
 *              one shorter if n is not a multiple of 64); Tq = ceil(nq/64) query
 *              tiles, Tk = ceil(nk/64) key tiles. With vsa_cubes, 4 x 4 x 4 cubes
 *              of the latent grid (as in the published method): cube (ct, cy, cx)
 *              holds the tokens with t/4 = ct, y/4 = cy, x/4 = cx; cubes are
 *              numbered cx fastest, then cy, then ct; Tq = Tk = ceil(grid_t/4) *
 *              ceil(grid_h/4) * ceil(grid_w/4). A grid side that is not a multiple
 *              of 4 makes its last cubes thinner (1 to 64 tokens): such a cube is a
 *              tile of its own tokens only (its mean divides by its token count,
 *              its keys are its tokens).
 *   coarse     mean of each tile of q and of k (float32 sum in ascending token order, then
 *              divided by the tile's token count); score(i, j) = sum over c of
 *              mean_q(i)[c] * mean_k(j)[c], each product and partial sum rounded
 *              to float32, c ascending (the positive softmax scale ranks nothing
 *              differently and is left out).
 *   selection  query tile i keeps the `keep` key tiles of highest score; equal
 *              scores keep the lower tile index; -0 equals +0 and NaN ranks
 *              lowest. keep = ceil((1 - sparsity) * Tk), at least 1.
 *   fine       every query of tile i attends over the keys of its kept tiles
 *              only, with the numerics of vdit_attn_fwd (fixed-reference softmax
 *              taken over the first kept tile).
 *
 * A plan for these calls has no key mask, no RoPE and no qk_int8 (UNSUPPORTED
 * otherwise); batch, both layouts and d = 64 or 128 work as for vdit_attn_fwd.
 * Limits: Tk <= 8192 and keep <= 4096 (UNSUPPORTED beyond); 1 <= keep <= Tk
 * (INVALID_ARG otherwise).
 *
 * vdit_vsa_keep: keep for a sparsity in [0, 1) (INVALID_ARG otherwise). Host only.
 * vdit_vsa_workspace_bytes: workspace bytes that every vsa call accepts for this
 *   keep: the attention workspace (v transposed; with vsa_cubes also k, both in
 *   cube order, one 64-slot tile per cube), then the kept tiles
 *   (int32 [B][head_count][Tq][keep]), the tile means (float32 [B][head_count][Tq][d]
 *   and [B][head_count][Tk][d]) and the coarse scores (float32
 *   [B][head_count][Tq][Tk]), each region 256-byte aligned. Host only.
 */
vdit_status_t vdit_vsa_keep(vdit_attn_t h, double sparsity, int32_t* keep);
vdit_status_t vdit_vsa_workspace_bytes(vdit_attn_t h, int32_t keep, size_t* bytes);

/*
 * Coarse stage: writes the kept key tiles of every (entry, head, query tile),
 * ascending, to `tiles` (device int32 [B][head_count][Tq][keep], 4-byte aligned).
 * q, k as for vdit_attn_fwd (N3HD: the packed tensor in q, k NULL); v is not
 * needed. workspace >= vdit_vsa_workspace_bytes(keep); `tiles` must not overlap
 * the inputs or the workspace (INVALID_ARG).
 */
vdit_status_t vdit_vsa_select(vdit_attn_t h, const void* q, const void* k, int32_t keep, int32_t* tiles,
                              void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Fine stage with caller-given tiles (device int32 [B][head_count][Tq][keep], e.g.
 * from vdit_vsa_select): prepares v into the workspace (>= vdit_attn_workspace_bytes)
 * and runs the block-sparse attention. A tile index outside [0, Tk) is clamped
 * into it (memory stays in bounds; the result then attends over the clamped
 * tile); listing a tile twice counts its keys twice. `tiles` must not overlap
 * out or the workspace. Other arguments as for vdit_attn_fwd.
 */
vdit_status_t vdit_vsa_attend(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t keep,
                              const int32_t* tiles, void* out, void* workspace, size_t workspace_bytes,
                              void* hip_stream);

/*
 * Both stages: vdit_vsa_select into the workspace, then vdit_vsa_attend.
 * workspace >= vdit_vsa_workspace_bytes(keep). Other arguments as for vdit_attn_fwd.
 */
vdit_status_t vdit_vsa_fwd(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t keep, void* out,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* Static, human-readable name of a status code (never NULL). */
const char* vdit_status_string(vdit_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* VDIT_ATTN_H */

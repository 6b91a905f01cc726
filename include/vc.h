/*
 * vc.h -- C ABI of the MI355X (gfx950) VC-Attention forward library (libvc.so).
 *
 * VC-Attention is FP8 (OCP E4M3) non-causal multi-head attention with two
 * additions, both defined in "VC-Attention: Value Smoothing and Softmax
 * Casting for Low-bit Attention", section "Abstract (arXiv)":
 *   - V-Smooth: value tokens of each (batch, head) are reordered by a light
 *     online clustering so each 128-token block holds similar tokens; only
 *     the residual after the block mean is quantised, and the mean is added
 *     back from the online-softmax row sum;
 *   - ExpCast-FP8: log-domain scores become E4M3 probability codes with one
 *     fused multiply-add.
 * The call shape ([B,S,H,128] or [S,H,128] FP16/BF16 in, BF16 out, head
 * dimension 128, non-causal, per-block Q/K and per-head V scales, an optional
 * V residual repair with a budget) follows "Open VC Attention", section
 * "Описание" (Description).
 *
 * Three calls make up one forward pass, all ordered on the caller's stream:
 *   vc_prepare_v     clustering, permutation, block means, E4M3 residual
 *   vc_prepare_qk    per-block E4M3 quantisation of Q and of K gathered
 *                    through the permutation of vc_prepare_v
 *   vc_attention_fwd the fused FP8 attention kernel (any number of times on
 *                    one prepared workspace)
 *
 * Memory and ownership: every pointer marked "device" is HIP device memory
 * owned by the caller; the library never allocates or frees device memory
 * and keeps no state between calls.  All intermediate results live in one
 * caller-provided workspace whose size and internal offsets come from
 * vc_workspace_layout (a host-only computation): vc_prepare_v needs
 * layout.total bytes, the other calls read only the regions before the
 * scratch region and need layout.scratch bytes.  Descriptors and option
 * structs are host memory, read during the call only.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  The library enqueues kernels and never synchronises; kernel
 * faults surface at the caller's next synchronisation.  The three calls
 * enqueue kernel launches only (no allocation, memset or copy, no host read
 * of device memory), so a caller with fixed shapes may record them into a
 * HIP graph and replay it; the graph keeps the buffers it was recorded with.
 *
 * Errors: every call validates its host-side arguments before it enqueues
 * any work; on failure it returns a non-zero vc_status, enqueues nothing,
 * and vc_last_error() returns a message (thread-local, valid until the next
 * call on the same thread).  VC_ERR_DEVICE means a HIP call or a kernel
 * launch failed; work already enqueued by that call may have run.
 *
 * Results are bit-deterministic for identical inputs and options.
 * Non-finite inputs are undefined behaviour.
 */
#ifndef VC_ATTN_VC_H
#define VC_ATTN_VC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VC_OK = 0,
  VC_ERR_ARG = 1,          /* null pointer, bad size, bad stride or option   */
  VC_ERR_UNSUPPORTED = 2,  /* D != 128, unsupported dtype or k, not gfx950   */
  VC_ERR_WORKSPACE = 3,    /* workspace smaller than vc_workspace_layout's   */
  VC_ERR_DEVICE = 4,       /* HIP runtime or kernel launch failure           */
  VC_STATUS_INT_RANGE_ = 0x7FFFFFFF  /* not a status: gives the enum the range of
                                        int32, so that vc_status_string is
                                        defined for any int a caller passes  */
} vc_status;

typedef enum { VC_F16 = 0, VC_BF16 = 1 } vc_dtype;

/* A [B,S,H,D] tensor view.  Element (b,s,h,d) is at
 * base + b*sB + s*sS + h*sH + d (strides in elements; D is contiguous).
 * D must be 128.  An [S,H,128] tensor is the view with B=1.
 * Base pointers and strides*2 bytes must be 16-byte aligned.  Supported
 * sizes: S <= 2^24, B*H <= 2^20, B and H each <= 65535, and
 * B*H*ceil(S/256) <= 2^23 - 1 (one attention launch; VC_ERR_UNSUPPORTED
 * otherwise). */
typedef struct {
  int32_t B, S, H, D;
  int32_t dtype;           /* vc_dtype */
  int32_t reserved;
  int64_t sB, sS, sH;
} vc_desc;

/* Residual formats ("Nunchux AI lanza VC-Attention kernel ...", paragraph 2:
 * the residual is kept in 8 bits (E4M3) or 4 bits (NVFP4)). */
typedef enum {
  VC_V_E4M3 = 0,           /* E4M3 codes with one scale per (b,h)                 */
  VC_V_MXFP4 = 1           /* OCP MXFP4 on gfx950: E2M1 codes, one power-of-two
                              (E8M0) scale per channel and run of 32 consecutive
                              permuted positions of a 128-key tile; no repair   */
} vc_v_format;

/* V-Smooth options. */
typedef struct {
  int32_t smooth;          /* 1: k-means reorder + block-mean subtraction;
                              0: identity order, no mean (plain per-head FP8 V) */
  int32_t k;               /* clusters per (b,h): 1 <= k <= min(S, 64)         */
  int32_t iters;           /* Lloyd iterations after the seeded init: 0..64     */
  int32_t v_format;        /* vc_v_format of the residual (0 = E4M3)            */
  uint64_t seed;           /* init offset: splitmix64(seed ^ (b*H+h))           */
  float repair_budget;     /* beta in [0,1): ceil(beta*S) repaired tokens per
                              (b,h); 0 disables repair                          */
  float reserved2;
} vc_v_opts;

/* Attention options. */
typedef struct {
  float sm_scale;          /* softmax scale > 0; 0 selects fp32(1/sqrt(128))   */
  int32_t reserved;
} vc_attn_opts;

/* Byte offsets of the workspace regions (all 256-byte aligned).  Per (b,h)
 * index bh = b*H + h; nblk = ceil(S/128); Sp = 128*nblk; nrep = ceil(beta*S);
 * nrep_pad = 128*ceil(nrep/128).
 *   q8      u8  [BH][nblk] tiles of 16384 B: Q codes, original token order
 *   q_scale f32 [BH][nblk]
 *   k8      u8  [BH][nblk] tiles: K codes, PERMUTED order (row p = token perm[p];
 *               VC_V_MXFP4: row r of tile b holds position 128b + mx(r), see below)
 *   k_scale f32 [BH][nblk]
 *   v8      u8  [BH][nblk] tiles: residual codes, permuted order, transposed
 *               (VC_V_MXFP4: the tile slot holds the E2M1 tile and its scales,
 *               see below)
 *   v_mean  f32 [BH][nblk][128] block means mu_b
 *   v_muop  u8  [BH][R][512] mu_b / s_v as bf16 high and low parts, laid
 *               out as matrix-core operands; R = 16*ceil((nblk+3)/16); row
 *               16G + 2*dt + h, lane l (8 bytes at 8*l): 4 bf16 values for
 *               channel 16*dt + l%16 and blocks 16G + 4*(l/16) + j, j=0..3,
 *               of the high (h=0) or low (h=1) part; zero past the last block
 *   hdr     per-(b,h) scalars, vc_head_hdr [BH]
 *   assign  i32 [BH][S] cluster id of each ORIGINAL token
 *   perm    i32 [BH][S] original token at permuted position p
 *   rep_pos i32 [BH][nrep_pad] repaired permuted positions, ascending; pad -1
 *   rep_k8  u8  [BH][nrep_pad/128] tiles: K codes of the repaired positions
 *   rep_ks  f32 [BH][nrep_pad] K block scale of each repaired position
 *   rep_e8  u8  [BH][nrep_pad/128] tiles: E4M3 residual error, transposed
 *   attn_part   vc_attention_fwd's partial results for work items it cuts
 *               along the key axis (the partial last round of workgroups,
 *               or every item of a launch with fewer items than compute
 *               units); empty when nothing is cut (always with repair) and
 *               for the short-launch form
 *   scratch     internal (k-means state, sort counters, repair scores)
 * Tile formats (16384 B, 128 rows x 128 columns of codes):
 *   row tile (q8, k8, rep_k8): the byte for (row r, column d) is at
 *     ((((r/16)*2 + (d%32)/16)*64 + (r%16) + 16*(d/32)) * 16) + d%16
 *   transposed tile (v8, rep_e8): the byte for (key j, channel d) is at
 *     ((((d/16)*2 + i/16)*64 + (d%16) + 16*g) * 16) + i%16,
 *     with g = (j%16)/4 and i = 4*(j/16) + j%4.
 *   MXFP4 tile (v8 with VC_V_MXFP4; 8704 of the slot's 16384 bytes): the
 *     permuted positions 32u .. 32u+31 of the tile form scale group u; the
 *     E2M1 code of (position j = 32u + n, channel d) is nibble n%2 (low
 *     first) of byte ((d/16)*64 + u*16 + d%16) * 16 + n/2, and the E8M0
 *     exponent byte (scale 2^(byte-127)) of the group (tile, d, u) is at
 *     8192 + (u*16 + d%16)*8 + d/16.  The K rows of an MXFP4 workspace are
 *     relabelled to match: row r = 16t + 4g + i of a k8 tile holds position
 *     mx(r) = 64*(t/4) + 16*g + 4*(t%4) + i of the tile (rows whose position
 *     is past S are zero).
 */
typedef struct {
  size_t total;
  size_t q8, q_scale, k8, k_scale, v8, v_mean, v_muop, hdr;
  size_t assign, perm, rep_pos, rep_k8, rep_ks, rep_e8, attn_part, scratch;
  int32_t nblk, nrep, nrep_pad, reserved;
} vc_ws_layout;

/* Per-(b,h) scalars in the workspace's hdr region. */
typedef struct {
  float v_scale;           /* s_v = a_R/448 (1 if a_R == 0)                     */
  float v_inv;             /* 448/a_R (1 if a_R == 0)                           */
  uint32_t v_amax_bits;    /* max|v| (float bits) over the head                 */
  uint32_t r_amax_bits;    /* a_R = max|R| (float bits) over the head           */
  int32_t shift;           /* k-means sketch scaling exponent                   */
  int32_t nrep;            /* repaired tokens for this head                     */
  float rep_scale;         /* s_e = a_e/448 (1 if a_e == 0)                     */
  uint32_t e_amax_bits;    /* a_e (float bits)                                  */
} vc_head_hdr;

/* Infrastructure (no passage of the pages defines it): host-only workspace
 * size and offsets for a V descriptor and options.  Only B, S, H, k and
 * repair_budget matter.  Returns VC_ERR_ARG or VC_ERR_UNSUPPORTED on invalid
 * shapes/options.  The layout depends on the options: every later call on
 * the workspace must pass the same options (vc_prepare_qk and
 * vc_attention_fwd read regions at these offsets). */
vc_status vc_workspace_layout(const vc_desc* vd, const vc_v_opts* opts, vc_ws_layout* out);

/* V-Smooth prepare ("VC-Attention: Value Smoothing and Softmax Casting for
 * Low-bit Attention", Abstract; "Nunchux AI lanza VC-Attention kernel ..."
 * paragraph 2: k-means per batch and head, mean of each 128-token block
 * subtracted, E4M3 residual; "Open VC Attention", Description: per-head V
 * scale, residual repair with a budget).
 *   vd, v   : V view (device), fp16/bf16, D == 128
 *   opts    : V-Smooth options (host)
 *   ws      : workspace (device), ws_bytes >= layout.total
 * Writes assign, perm, v8, v_mean, v_muop, hdr and the repair set. */
vc_status vc_prepare_v(const vc_desc* vd, const void* v, const vc_v_opts* opts,
                       void* ws, size_t ws_bytes, void* stream);

/* Allocation-free V prepare, for callers that cannot allocate device memory
 * (code being recorded into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and results as vc_prepare_v, but the
 * internal scratch (k-means centroids and sums, sort counters, repair
 * scores: layout.total - layout.scratch bytes) is a static device array of
 * VC_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, so `ws` needs only layout.scratch bytes -- the
 * prepared products, which is all vc_prepare_qk and vc_attention_fwd read.
 * Returns VC_ERR_UNSUPPORTED when the shape needs more scratch than the
 * array holds.  Calls no hipMalloc or hipFree.  Every call on one GPU shares
 * that GPU's array and each call initialises the parts it reads: calls that
 * overlap on one GPU (other streams or threads) race, so the caller
 * serialises them. */
#define VC_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
vc_status vc_prepare_v_noalloc(const vc_desc* vd, const void* v, const vc_v_opts* opts, void* ws,
                               size_t ws_bytes, void* stream);

/* Q/K prepare ("Open VC Attention", Description: per-block Q/K scales).
 * Q is quantised in its original order; K is gathered through perm (written
 * by vc_prepare_v on the same workspace, earlier on the same stream) so that
 * keys and values stay paired.  Per 128-token block: scale = amax/448,
 * code = E4M3(x * (448/amax)).  qd and kd must agree on B, S, H, D, and with
 * the V that vc_prepare_v prepared; `opts` must be the options it was
 * prepared with (the workspace offsets depend on them, and an MXFP4
 * workspace stores K rows in its relabelled order).  A permutation entry
 * outside [0, S) -- a workspace not prepared for this shape -- gives zero K
 * rows, never a read outside the K tensor.
 *   ws      : workspace (device), ws_bytes >= layout.scratch */
vc_status vc_prepare_qk(const vc_desc* qd, const void* q, const vc_desc* kd, const void* k,
                        const vc_v_opts* opts, void* ws, size_t ws_bytes, void* stream);

/* Fused attention ("VC-Attention: Value Smoothing and Softmax Casting for
 * Low-bit Attention", Abstract; "Hugging Face Introduces VC-Attention ...",
 * Technical Breakthroughs and Core Innovations).  For every query and every
 * 128-key tile in ascending order: FP8 MFMA scores, integer log2 running
 * maximum, ExpCast E4M3 probability codes, row sum, exact power-of-two
 * rescale, FP8 MFMA P.V, block-mean restore; then the repair tiles; output
 * out = (s_v*O + s_e*O_rep)/l rounded to bf16.
 *   od      : output view (device memory `out`), dtype must be VC_BF16, same
 *             B, S, H as the prepared inputs; rows stay in the original
 *             query order
 *   opts    : the V options the workspace was prepared with -- the same
 *             struct values: the workspace offsets and the V tile format
 *             depend on them, and nothing on the device records them, so
 *             other options read other regions (within the workspace, never
 *             outside it) and give a wrong result
 *   aopts   : may be NULL (defaults)
 *   ws      : a workspace prepared by vc_prepare_v and vc_prepare_qk,
 *             ws_bytes >= layout.scratch
 * Work items are (b,h) and a pair of 128-query blocks, one workgroup each;
 * the items of a partial last round of workgroups (or all of them, when
 * there are fewer items than compute units) are cut along the key axis and
 * their pieces merged exactly (powers of two) by a second kernel, which uses
 * the workspace's attn_part region.  Workspaces with a repair set are not
 * cut.  A short launch -- at most 256 query blocks in all, 2048 < S <= 4096,
 * no repair set -- runs instead one workgroup per (b,h) and query block with
 * its key tiles in two halves merged inside the workgroup (the same
 * arithmetic; no attn_part, no second kernel). */
vc_status vc_attention_fwd(const vc_desc* od, void* out, const vc_v_opts* opts,
                           const vc_attn_opts* aopts, const void* ws, size_t ws_bytes,
                           void* stream);

/* Infrastructure (no passage of the pages defines them): status names and
 * the calling thread's last error message.  Static strings; never NULL. */
const char* vc_status_string(vc_status s);
const char* vc_last_error(void);

/* Infrastructure (no passage): library version, e.g. "0.1.0". */
const char* vc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VC_ATTN_VC_H */

// vc_kernels.hpp -- internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vc.h"

namespace vc {

// Threads per attention workgroup (8 waves, two 128-query blocks).  A launch
// holds at most 2^32 - 1 threads, so at most kMaxAttnWorkgroups workgroups.
constexpr int kAttnThreadsPerWg = 512;
constexpr int64_t kMaxAttnWorkgroups = 0xFFFFFFFFll / kAttnThreadsPerWg;

// A [B,S,H,128] fp16/bf16 view (element strides; D contiguous).
struct TensorArg {
  const void* p;
  int64_t sB, sS, sH;
  int dtype;
};

// Typed pointers into one workspace.
struct WsPtrs {
  uint8_t *q8, *k8, *v8, *rep_k8, *rep_e8, *v_muop;
  float *q_scale, *k_scale, *v_mean, *rep_ks;
  vc_head_hdr* hdr;
  int32_t *assign, *perm, *rep_pos;
  int32_t* cent;
  int64_t* csum;    // per-cluster sketch sums: up to 255 * S in magnitude
  int32_t *ccount, *chunk_hist, *chunk_off, *cnorm;
  uint8_t* cent_op;
  double* rep_norm;
  int nblk, nrep, nrep_pad;
};

struct AttnArgs {
  const uint8_t* q8;
  const float* q_scale;
  const uint8_t* k8;
  const float* k_scale;
  const uint8_t* v8;
  const uint8_t* v_muop;
  const vc_head_hdr* hdr;
  const uint8_t* rep_k8;
  const float* rep_ks;
  const uint8_t* rep_e8;
  uint16_t* out;
  int64_t osB, osS, osH;
  int S, H, nblk, nrep_pad, whole;   // whole: work items run whole (the first launch's workgroups)
  float sm_scale;
  int v_format;       // vc_v_format of the residual tiles in v8
};

// The cut items (attn_split): tail_wg workgroups run the `tail` items after
// the whole ones in runs of `per` 16-tile groups (ngrp per item), with
// partial slots at `part`, then the merge launch; or, with `halves`, the
// short-launch form in place of all of that.
struct AttnTail {
  int tail, tail_wg, per, ngrp;
  float* part;
  int halves;         // the short-launch form (attn_split): its B*H*nblk workgroups, or 0
  int ka;             // its key halves: tiles [0, ka) and [ka, nblk)
};

hipError_t launch_prepare_v(const TensorArg& v, int B, int S, int H, const vc_v_opts& o, const WsPtrs& ws,
                            hipStream_t st);
hipError_t launch_prepare_qk(const TensorArg& q, const TensorArg& k, int B, int S, int H, int v_format,
                             const WsPtrs& ws, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, const AttnTail& tl, hipStream_t st);

}  // namespace vc

// vc_attn.hip -- fused VC-Attention forward kernel for gfx950 (MI355X).
//
// Method ("VC-Attention: Value Smoothing and Softmax Casting for Low-bit
// Attention", Abstract; "Hugging Face Introduces VC-Attention ...",
// Technical Breakthroughs and Core Innovations): both attention products run
// on FP8 (E4M3) matrix cores; between them the log-domain score becomes an
// E4M3 probability code with one fused multiply-add (ExpCast), the online
// softmax keeps the row sum, and V-Smooth's block mean is restored from that
// tile's row sum.
//
// Numerics per query row and 128-key tile b (ascending):
//   acc   = Q8 . K8^T                       FP8 MFMA, fp32 accumulate
//   sigma = ((s_q * s_k[b]) * sm_scale) * log2(e)      fp32
//   M'    = max(M, ceil(max_j acc * sigma))  integer log2 running maximum
//   code  = sat_u8(rne(fma(acc, 8*sigma, 120 - 8*M'))) = E4M3 byte of P
//   r     = sum_j P (row sum; MFMA against a tile of E4M3 ones)
//   l     = 2^(M-M') * l + r
//   O     = 2^(M-M') * O + P . V8 + r * mu_b / s_v
// then the repair tiles add P_rep . E8 (scale s_e, codes against the final
// M, not added to l) and out = bf16(s_v * (O + (s_e/s_v) O_rep) / l).
//
// Layout and schedule:
//   * one workgroup = 4 waves = one 128-query block of one (b,h); wave w owns
//     queries 32w..32w+31 as two 16-query sub-tiles;
//   * transposed products: S^T = K.Q^T with v_mfma_f32_16x16x128_f8f6f4, so
//     each lane holds one query column; row max and row sum stay in-lane
//     apart from one 4-lane combine;
//   * the S^T accumulator bytes (keys 16t+4g+i for lane group g) are exactly
//     the B-operand slots of O^T = V^T.P^T, so P never leaves registers; the
//     prepare stage stores V8 in that slot order;
//   * K and V tiles (16 KB each) are staged in LDS, double buffered, loaded
//     with 16-byte coalesced global loads, one barrier per tile;
//   * workgroup ids are remapped so each XCD runs consecutive query blocks of
//     the same head: its 4 MB L2 then serves the K/V stream to all of them.
#include "vc_common.hpp"
#include "vc_kernels.hpp"

namespace vc {

constexpr int kAttnThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = blgp = 0: both operands OCP E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i ld_op_lds(const uint8_t* base, int sub, int lane) {
  // operand for sub-tile `sub`: two 16-byte halves 1 KB apart
  const uint4 lo = *reinterpret_cast<const uint4*>(base + ((sub * 2) * 64 + lane) * 16);
  const uint4 hi = *reinterpret_cast<const uint4*>(base + ((sub * 2 + 1) * 64 + lane) * 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

__device__ __forceinline__ v8i ld_op_global(const uint8_t* base, int sub, int lane) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + ((sub * 2) * 64 + lane) * 16);
  const uint4 hi = *reinterpret_cast<const uint4*>(base + ((sub * 2 + 1) * 64 + lane) * 16);
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// ExpCast of one 16x16 accumulator (4 keys per lane) into one packed dword.
__device__ __forceinline__ uint32_t expcast4(const v4f& s, float s8, float c) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s[0], s8, c), 0, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s[1], s8, c), 1, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s[2], s8, c), 2, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s[3], s8, c), 3, w);
  return w;
}

__device__ __forceinline__ float max4(const v4f& s) { return fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])); }

__global__ void __launch_bounds__(kAttnThreads, 2) k_vc_attn_fwd(AttnArgs a) {
  __shared__ __align__(16) uint8_t kv[2][2][kTileBytes];   // [buffer][K, V]
  __shared__ __align__(16) float mus[2][kD];

  // XCD-aware order: hardware deals workgroup ids round-robin over 8 XCDs;
  // give XCD x a contiguous range of (head, query-block) work items.
  const int total = a.total_wg;
  const int wg = blockIdx.x, xcd = wg & 7, idx = wg >> 3;
  const int per = total >> 3, rem = total & 7;
  const int logical = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int nblk = a.nblk;
  const int bh = logical / nblk, qb = logical - bh * nblk;
  const int b = bh / a.H, h = bh - b * a.H;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int S = a.S;

  // Q^T operands for this wave's two 16-query sub-tiles (kept in registers)
  const uint8_t* qtile = a.q8 + (static_cast<int64_t>(bh) * nblk + qb) * kTileBytes;
  v8i qop[2];
  qop[0] = ld_op_global(qtile, 2 * w, lane);
  qop[1] = ld_op_global(qtile, 2 * w + 1, lane);
  const float s_q = a.q_scale[static_cast<int64_t>(bh) * nblk + qb];
  const float* ks = a.k_scale + static_cast<int64_t>(bh) * nblk;

  v8i ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;   // E4M3 1.0
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};

  float M[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.0f, 0.0f};
  v4f O[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt][0] = O[dt][1] = zero;

  const uint8_t* kbase = a.k8 + static_cast<int64_t>(bh) * nblk * kTileBytes;
  const uint8_t* vbase = a.v8 + static_cast<int64_t>(bh) * nblk * kTileBytes;
  const float* mbase = a.v_meanp + static_cast<int64_t>(bh) * nblk * kD;

  // staging registers for the next K/V tile and its block means
  uint4 stk0, stk1, stk2, stk3, stv0, stv1, stv2, stv3;
  float4 stm = make_float4(0, 0, 0, 0);
#define VC_GLOAD(kb_)                                                                               \
  do {                                                                                              \
    const uint4* ksrc_ = reinterpret_cast<const uint4*>(kbase + static_cast<int64_t>(kb_) * kTileBytes); \
    const uint4* vsrc_ = reinterpret_cast<const uint4*>(vbase + static_cast<int64_t>(kb_) * kTileBytes); \
    stk0 = ksrc_[tid];                                                                              \
    stk1 = ksrc_[tid + kAttnThreads];                                                               \
    stk2 = ksrc_[tid + 2 * kAttnThreads];                                                           \
    stk3 = ksrc_[tid + 3 * kAttnThreads];                                                           \
    stv0 = vsrc_[tid];                                                                              \
    stv1 = vsrc_[tid + kAttnThreads];                                                               \
    stv2 = vsrc_[tid + 2 * kAttnThreads];                                                           \
    stv3 = vsrc_[tid + 3 * kAttnThreads];                                                           \
    if (tid < kD / 4) stm = reinterpret_cast<const float4*>(mbase + static_cast<int64_t>(kb_) * kD)[tid]; \
  } while (0)
#define VC_LSTORE(buf_)                                                                             \
  do {                                                                                              \
    uint4* kd_ = reinterpret_cast<uint4*>(kv[buf_][0]);                                             \
    uint4* vd_ = reinterpret_cast<uint4*>(kv[buf_][1]);                                             \
    kd_[tid] = stk0;                                                                                \
    kd_[tid + kAttnThreads] = stk1;                                                                 \
    kd_[tid + 2 * kAttnThreads] = stk2;                                                             \
    kd_[tid + 3 * kAttnThreads] = stk3;                                                             \
    vd_[tid] = stv0;                                                                                \
    vd_[tid + kAttnThreads] = stv1;                                                                 \
    vd_[tid + 2 * kAttnThreads] = stv2;                                                             \
    vd_[tid + 3 * kAttnThreads] = stv3;                                                             \
    if (tid < kD / 4) reinterpret_cast<float4*>(mus[buf_])[tid] = stm;                              \
  } while (0)

  VC_GLOAD(0);
  VC_LSTORE(0);
  __syncthreads();

  for (int kb = 0; kb < nblk; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nblk) VC_GLOAD(kb + 1);

    // ---- scores S^T = K . Q^T (16 MFMAs) ----
    v4f sc[8][2];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const v8i kop = ld_op_lds(kv[buf][0], t, lane);
      sc[t][0] = mfma_fp8(kop, qop[0], zero);
      sc[t][1] = mfma_fp8(kop, qop[1], zero);
    }
    if ((kb + 1) * kBlock > S) {            // ragged last tile: mask padded keys
      const int kval = S - kb * kBlock;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * t + 4 * g + i >= kval) sc[t][0][i] = sc[t][1][i] = -INFINITY;
    }
    const float sigma = ((s_q * ks[kb]) * a.sm_scale) * kLog2e;
    const float s8 = 8.0f * sigma;

    // ---- integer running max, rescale, ExpCast ----
    v8i P[2];
    float alpha[2];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      float mx = max4(sc[0][qi]);
#pragma unroll
      for (int t = 1; t < 8; ++t) mx = fmaxf(mx, max4(sc[t][qi]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(M[qi], ceilf(mx * sigma));
      alpha[qi] = M[qi] == -INFINITY ? 0.0f : ldexpf(1.0f, static_cast<int>(fmaxf(M[qi] - mn, -160.0f)));
      M[qi] = mn;
      const float c = 120.0f - 8.0f * mn;
#pragma unroll
      for (int t = 0; t < 8; ++t) P[qi][t] = static_cast<int>(expcast4(sc[t][qi], s8, c));
    }
    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        l[qi] *= alpha[qi];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) O[dt][qi] *= alpha[qi];
      }
    }

    // ---- row sums on the matrix core: ones(16x128) . P^T ----
    float r[2];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      const v4f rs = mfma_fp8(ones, P[qi], zero);
      r[qi] = rs[0];
      l[qi] += r[qi];
    }

    // ---- O^T += V^T . P^T (16 MFMAs) and block-mean restore ----
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const v8i vop = ld_op_lds(kv[buf][1], dt, lane);
      O[dt][0] = mfma_fp8(vop, P[0], O[dt][0]);
      O[dt][1] = mfma_fp8(vop, P[1], O[dt][1]);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const float4 mu = *reinterpret_cast<const float4*>(&mus[buf][16 * dt + 4 * g]);
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        O[dt][qi][0] = fmaf(r[qi], mu.x, O[dt][qi][0]);
        O[dt][qi][1] = fmaf(r[qi], mu.y, O[dt][qi][1]);
        O[dt][qi][2] = fmaf(r[qi], mu.z, O[dt][qi][2]);
        O[dt][qi][3] = fmaf(r[qi], mu.w, O[dt][qi][3]);
      }
    }

    if (kb + 1 < nblk) VC_LSTORE(buf ^ 1);
    __syncthreads();
  }

#undef VC_GLOAD
#undef VC_LSTORE
  const vc_head_hdr hd = a.hdr[bh];

  // ---- residual repair tiles (codes against the final maximum) ----
  if (a.nrep_pad > 0) {
    const int nrep = hd.nrep;
    const float fe = hd.rep_scale / hd.v_scale;
    const uint8_t* rk = a.rep_k8 + static_cast<int64_t>(bh) * a.nrep_pad * kD;
    const uint8_t* re = a.rep_e8 + static_cast<int64_t>(bh) * a.nrep_pad * kD;
    const float* rks = a.rep_ks + static_cast<int64_t>(bh) * a.nrep_pad;
    const float sq = s_q * a.sm_scale;
    for (int rt = 0; rt < a.nrep_pad / kBlock; ++rt) {
      v8i P[2];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const v8i kop = ld_op_global(rk + static_cast<int64_t>(rt) * kTileBytes, t, lane);
        const v4f s0 = mfma_fp8(kop, qop[0], zero);
        const v4f s1 = mfma_fp8(kop, qop[1], zero);
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = rt * kBlock + 16 * t + 4 * g + i;
          const float sig = ((s_q * rks[j]) * a.sm_scale) * kLog2e;
          const float s8j = j < nrep ? 8.0f * sig : 0.0f;
          const float c0 = j < nrep ? 120.0f - 8.0f * M[0] : -1.0f;
          const float c1 = j < nrep ? 120.0f - 8.0f * M[1] : -1.0f;
          w0 = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s0[i], s8j, c0), i, w0);
          w1 = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s1[i], s8j, c1), i, w1);
        }
        P[0][t] = static_cast<int>(w0);
        P[1][t] = static_cast<int>(w1);
      }
      (void)sq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v8i eop = ld_op_global(re + static_cast<int64_t>(rt) * kTileBytes, dt, lane);
        const v4f o0 = mfma_fp8(eop, P[0], zero);
        const v4f o1 = mfma_fp8(eop, P[1], zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          O[dt][0][i] = fmaf(fe, o0[i], O[dt][0][i]);
          O[dt][1][i] = fmaf(fe, o1[i], O[dt][1][i]);
        }
      }
    }
  }

  // ---- epilogue: out = bf16(s_v * O / l), original query order ----
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int q = qb * kBlock + 16 * (2 * w + qi) + l16;
    if (q < S) {
      const float f = hd.v_scale / l[qi];
      uint16_t* orow = a.out + b * a.osB + static_cast<int64_t>(q) * a.osS + h * a.osH;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint32_t lo = f32_to_bf16_bits(O[dt][qi][0] * f) | (f32_to_bf16_bits(O[dt][qi][1] * f) << 16);
        const uint32_t hi = f32_to_bf16_bits(O[dt][qi][2] * f) | (f32_to_bf16_bits(O[dt][qi][3] * f) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g) = make_uint2(lo, hi);
      }
    }
  }
}

hipError_t launch_attention(const AttnArgs& a, int BH, hipStream_t st) {
  (void)BH;
  hipLaunchKernelGGL(k_vc_attn_fwd, dim3(a.total_wg), dim3(kAttnThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace vc

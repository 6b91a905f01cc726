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
// With the 4-bit V residual the P.V MFMA takes block scales anyway, so O, l
// and the row sums there stay relative to an anchor A <= M and the codes'
// MFMA scale 2^(M-A) replaces the rescale (exact: powers of two).
//
// Layout and schedule:
//   * one workgroup = 8 waves = two 128-query blocks of one (b,h); wave w
//     owns 32 queries of block w/4 as two 16-query sub-tiles;
//   * transposed products: S^T = K.Q^T with v_mfma_f32_16x16x128_f8f6f4, so
//     each lane holds one query column; row max and row sum stay in-lane
//     apart from one cross-row combine;
//   * the S^T accumulator bytes (keys 16t+4g+i for lane group g) are exactly
//     the B-operand slots of O^T = V^T.P^T, so P never leaves registers; the
//     prepare stage stores V8 in that slot order;
//   * K and V tiles (16 KB each) stream through 4-deep LDS rings, copied
//     straight from global memory into LDS three steps ahead, one barrier
//     per step;
//   * scores run one tile ahead of their cast: step kb does the P.V MFMAs
//     of tile kb and then the score MFMAs of tile kb+2, and under them the
//     vector ALU casts tile kb+1's scores (computed by the previous step)
//     against the maximum after tile kb+1 and keeps the running max of tile
//     kb+2's; so a code is cast once, against the final maximum of its own
//     tile.  Whether a maximum rose is decided from each lane's partial
//     maximum; the cross-row combine runs only when one did;
//   * the block-mean restore r_b * mu_b/s_v is deferred: each tile's row sum
//     is kept (and rescaled with O), and every 16 tiles the sums meet the
//     prepared mu/s_v operands in 16x16x16 bf16 MFMAs (high/low bf16 parts,
//     three products), instead of 64 fp32 FMAs per tile on the VALU;
//   * workgroup ids are remapped so each XCD runs consecutive query blocks of
//     the same head: its 4 MB L2 then serves the K/V stream to all of them;
//   * one workgroup fills a compute unit (its LDS), so work items run in
//     rounds of 256.  The items of a partial last round (all of them, when a
//     launch has fewer) are cut along the key axis into pieces of whole
//     16-tile groups (k_vc_attn_tail); each piece leaves unnormalised O, row
//     sums and its reference exponent in a partial slot, and k_vc_attn_merge
//     adds an item's pieces with power-of-two weights, the online softmax's
//     own rescale.
#include <type_traits>

#include "vc_common.hpp"
#include "vc_kernels.hpp"

namespace vc {

constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = kAttnThreadsPerWg;   // two 128-query blocks per workgroup
static_assert(kAttnThreads == 64 * kAttnWaves, "one workgroup is kAttnWaves waves");
constexpr float kLog2e = 1.44269504088896340736f;
// Four E4M3 1.0 codes: the ones operand of the row-sum MFMA.
constexpr int kOnes4 = 0x38383838;

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = blgp = 0: both operands OCP E4M3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// Same with a power-of-two scale on the B operand's columns: byte QI of se
// is the E8M0 exponent (127 = 1.0) that every lane applies to its column;
// byte 2 of se is 127, the scale of A (one register serves both).
template <int QI>
__device__ __forceinline__ v4f mfma_fp8_sb(const v8i& a, const v8i& b, const v4f& c, int se) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 2, se, QI, se);
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

// Same, from a pointer that already includes the lane's 16-byte offset:
// the sub-tile offsets then fit the instruction's immediate field.
__device__ __forceinline__ v8i ld_op_lds_at(const uint8_t* p, int sub) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p + (sub * 2) * 1024);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + (sub * 2 + 1) * 1024);
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

// Tiles go from global memory straight into LDS with buffer loads (the
// buffer form: the compiler tracks these copies on the vector-memory counter
// only, so waits for LDS reads issued after a copy stay partial).  Every
// lane moves 16 bytes to LDS address M0 + 16*lane; a per-head buffer
// resource bounds every copy (an offset past it reads zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw 32-bit untyped access (the CDNA3/CDNA4 setting)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, 0,
                                           0, 0);
}
// The same with the wave-uniform part of the offset in the scalar offset
// field, so the lane's part (16 * lane, one kept register) needs no vector
// arithmetic.  Callers keep soff + voff inside the tile range by
// construction (clamped tile indices).
__device__ __forceinline__ void copy16_to_lds_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                uint8_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff,
                                           static_cast<int>(soff), 0, 0);
}
constexpr int kDmaPerTile = kTileBytes / (16 * kAttnThreads);   // copy instructions per 16 KB tile
// LDS ring depth for K and for V tiles; copies run kStages-1 tiles ahead.
constexpr int kStages = 4;
// V tile formats (VF = vc_v_format): E4M3, 16 KB; MXFP4, 8 KB of E2M1 codes
// then 512 B of scale exponents (8 per lane), copied with a 1 KB landing zone.
constexpr int kFp4CodeBytes = 8192;
template <int VF> struct VTile {
  static constexpr int kBytes = VF ? kFp4CodeBytes + 1024 : kTileBytes;       // LDS buffer
  static constexpr int kDma = VF ? kFp4CodeBytes / (16 * kAttnThreads) : kDmaPerTile;   // code copies per wave
};
// Copy instructions per step: every wave copies its share of one K and one
// V tile; wave 0 also copies the K tile's scale and one restore-operand row
// (and, for MXFP4, wave 1 the V tile's scales).
template <int VF> constexpr int kDmaPerStep = kDmaPerTile + VTile<VF>::kDma;
// A K buffer: the K tile, then its scale, written by every lane of a 4-byte
// copy (256 bytes).
constexpr int kKBufBytes = kTileBytes + 256;
// A restore-operand group buffer: 16 rows of 512 bytes plus the landing room
// of lanes 32..63 of the last row's copy (they carry the next row).
constexpr int kGrpBytes = kMuOpGroup * kMuOpRowBytes + kMuOpRowBytes;

// End of a tile step: every wave waits until at most the (kStages-2) *
// kDmaPerStep newest of its copies may still be in flight, and until its LDS
// reads have returned; then the workgroup barrier.  The copies of a step are
// always its last vector-memory instructions and every wave issues at least
// kDmaPerStep of them per step, so the count means that every copy issued
// kStages-2 or more steps earlier has landed (waves with extra copies -- a K
// scale, a restore-operand row, MXFP4 scales -- only finish earlier).  One
// count for all waves keeps the compiler's own wait analysis exact.
template <int VF>
__device__ __forceinline__ void step_barrier() {
  // s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14.
  // Written as a builtin so the compiler's own wait insertion knows that
  // every older copy has landed after this point.
  constexpr int kVm = (kStages - 2) * kDmaPerStep<VF>;
  static_assert(kVm < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((kVm & 15) | (7 << 4) | (0 << 8) | ((kVm >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

// The probability cast of two scores into bytes 2h, 2h+1 of a packed code
// dword, with the per-tile scale a and the per-row constant b:
//   ExpCast:  code = sat_u8(rne(fma(acc, a, b))), a = 8*sigma, b = 120 - 8*M
// (one FMA and one byte conversion per score).  A build with
// VC_ABLATION_EXP_CAST instead takes the FP32 exponential that ExpCast
// replaces ("VC-Attention: Value Smoothing and Softmax Casting for Low-bit
// Attention", Abstract): p = 2^fma(acc, a, b) with a = sigma, b = 8 - M (so
// p = 256 * 2^(acc*sigma - M)) on the transcendental unit, then an E4M3
// cast (round to nearest even) -- for measuring what the cast saves; it is
// not the method.
#ifndef VC_ABLATION_EXP_CAST
__device__ __forceinline__ float cast_scale(float sigma) { return 8.0f * sigma; }
__device__ __forceinline__ float cast_const(float m) { return 120.0f - 8.0f * m; }
__device__ __forceinline__ uint32_t pcast2(float x0, float x1, float a, float b, int h, uint32_t w) {
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x0, a, b), 2 * h, w);
  return __builtin_amdgcn_cvt_pk_u8_f32(fmaf(x1, a, b), 2 * h + 1, w);
}
#else
__device__ __forceinline__ float cast_scale(float sigma) { return sigma; }
__device__ __forceinline__ float cast_const(float m) { return 8.0f - m; }
__device__ __forceinline__ uint32_t pcast2(float x0, float x1, float a, float b, int h, uint32_t w) {
  const float p0 = __builtin_amdgcn_exp2f(fmaf(x0, a, b));
  const float p1 = __builtin_amdgcn_exp2f(fmaf(x1, a, b));
  // the word select of the conversion is an immediate
  return static_cast<uint32_t>(h ? __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, static_cast<int>(w), true)
                                 : __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, static_cast<int>(w), false));
}
// two scores with their own scales and constants (the repair tiles, whose
// keys each carry a scale) into bytes 2h, 2h+1 of w
__device__ __forceinline__ uint32_t pcast2v(float x0, float x1, const float (&a)[2], const float (&b)[2], int h,
                                            uint32_t w) {
  const float p0 = __builtin_amdgcn_exp2f(fmaf(x0, a[0], b[0]));
  const float p1 = __builtin_amdgcn_exp2f(fmaf(x1, a[1], b[1]));
  return static_cast<uint32_t>(h ? __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, static_cast<int>(w), true)
                                 : __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, static_cast<int>(w), false));
}
// cast constant that sends a score to code 0 (masked repair slots)
constexpr float kCastOff = -200.0f;
#endif

// Cast of one 16x16 accumulator (4 keys per lane) into one packed dword.
__device__ __forceinline__ uint32_t expcast4(const v4f& s, float a, float b) {
  uint32_t w = pcast2(s[0], s[1], a, b, 0, 0u);
  return pcast2(s[2], s[3], a, b, 1, w);
}

__device__ __forceinline__ float max4(const v4f& s) { return fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])); }
// running max over 4 more values as two 3-input maxima
__device__ __forceinline__ float max_acc4(float m, const v4f& s) { return fmaxf(fmaxf(fmaxf(fmaxf(m, s[0]), s[1]), s[2]), s[3]); }

// Large finite stand-in for -infinity for masked scores (the kernel is built
// without NaN/IEEE canonicalisation and never forms a NaN; the maximum of a
// fully masked tile times sigma may round to -infinity, which the comparisons
// and fmaxf against a finite M handle).
constexpr float kNegBig = -3.0e38f;

// Per-wave online-softmax state for two 16-query sub-tiles.
struct SoftState {
  float M[2];      // integer log2 running maximum (kNegBig before the first tile)
  float l[2];      // running row sum
  float cq[2];     // cast_const(M) (120 - 8*M): the cast constant for the current maximum
  // MXFP4 V: O, l and the restore weights are held relative to an anchor
  // maximum A <= M per query instead of M itself: byte qi of se is
  // 127 + (M - A), the E8M0 scale that the P.V and row-sum MFMAs put on codes
  // cast against M (byte 2 is 127, the ones operand's scale).  A rise of M
  // then changes one byte instead of rescaling every accumulator; A moves up
  // to M (with the rescale) only once M - A would pass kAnchorSpan.  E4M3 V
  // keeps A = M (the unscaled MFMA is the faster one there) and se at 127.
  int se;
};
// Largest M - A kept before the accumulators are rescaled: O stays below
// 2^(kAnchorSpan + 41) (codes <= 256, |V| <= 448, <= 2^24 keys), far from
// the FP32 limit.
constexpr int kAnchorSpan = 64;

// Half the ExpCast of an accumulator (keys i0, i0+1 of one 16-key
// sub-tile): two FMAs and two conversions into the packed code dword.
__device__ __forceinline__ void cast_half(const v4f& s, int i0, float s8, float c, uint32_t& w) {
  w = pcast2(s[i0], s[i0 + 1], s8, c, i0 >> 1, w);
}
// Running max over one accumulator: two 3-input maxima.
__device__ __forceinline__ void max_acc(const v4f& s, float& mx) {
  mx = fmaxf(fmaxf(mx, s[0]), s[1]);
  mx = fmaxf(fmaxf(mx, s[2]), s[3]);
}

// The V operand of channel sub-tile dt: E4M3, 32 bytes per lane; MXFP4, 16
// bytes of E2M1 codes per lane (the matrix core reads four registers).
template <int VF>
__device__ __forceinline__ v8i ld_vop(const uint8_t* vl, int dt) {
  if (VF == 0) return ld_op_lds_at(vl, dt);
  const uint4 c = *reinterpret_cast<const uint4*>(vl + dt * 1024);
  v8i r = {static_cast<int>(c.x), static_cast<int>(c.y), static_cast<int>(c.z), static_cast<int>(c.w), 0, 0, 0, 0};
  return r;
}
// O^T[dt] += V^T[dt] . P^T for query sub-tile QI, with byte QI of se on P
// (codes relative to the anchor, SoftState::se); for MXFP4 also the lane's
// E8M0 scale of this dt (byte dt%4 of vsc[dt/4]) on V.
// (dt is a constant once the caller's loop is unrolled; the byte select is
// an immediate of the instruction, hence the switch)
template <int VF, int QI>
__device__ __forceinline__ v4f pv_mfma(const v8i& vop, const v8i& p, const v4f& o, const uint32_t (&vsc)[2], int dt,
                                       int se) {
  if (VF == 0) return mfma_fp8(vop, p, o);
  const int sc = static_cast<int>(vsc[dt >> 2]);
  switch (dt & 3) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, p, o, 4, 0, 0, sc, QI, se);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, p, o, 4, 0, 1, sc, QI, se);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, p, o, 4, 0, 2, sc, QI, se);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, p, o, 4, 0, 3, sc, QI, se);
  }
}

// The new maximum of query sub-tile qi from the held tile's partial row
// maxima: the cross-row combine, the integer ceiling and the cast constant.
// Did any row's maximum rise?  ceil(fl(m*sigma)) > M for an integer M
// exactly when fl(m*sigma) > M, and fl(m*sigma) is monotone in m, so each
// lane's partial maximum decides without the cross-row combine, which then
// runs only when one did (a wave-uniform branch).  Returns that decision
// (wave-uniform); only then is d = how far each row rose (>= 0, an integer)
// set, and some row's d is > 0.
__device__ __forceinline__ bool new_max(SoftState& st, int qi, float mh, float sig, float& d) {
  if (__builtin_expect(__any(mh * sig > st.M[qi]), 0)) {
    const float mn = fmaxf(st.M[qi], ceilf(max_over_rows(mh) * sig));
    d = mn - st.M[qi];
    st.M[qi] = mn;
    st.cq[qi] = cast_const(mn);
    return true;
  }
  return false;
}

// The matrix-core work of one step kb, in two halves.  First the P.V MFMAs
// of tile kb (V in LDS, codes P of tile kb) and its two row-sum MFMAs
// (codes against a tile of E4M3 ones); under them the vector ALU finishes
// the running max of tile kb+1's scores (sh, computed by the previous step,
// with per-lane partial maxima mh), takes the maximum after tile kb+1 and
// starts the ExpCast of those scores against it into Pn.  Then the score
// MFMAs of tile kb+2 (K in LDS, both query sub-tiles) into sn; under them
// the rest of the cast, the per-lane running max (mn) of the new scores
// (sub-tile 7's max is left to the next step) and tile kb's row sums into l
// and into its restore-weight slot rr.  A tile's maximum is thus
// known before its codes are cast, so no cast is ever redone; and the held
// scores are cast before the new ones arrive, so the two sets share
// registers.  Each MFMA is followed by a few of these instructions (a score
// sub-tile is read two MFMAs after it was issued, so its result is ready);
// order and placement are fixed with scheduling barriers.  Operands are
// read from LDS two sub-tiles ahead; copy parts 0..5 go out spread over the
// step.
template <int VF, typename Copies>
__device__ __forceinline__ void mfma_phase(const uint8_t* ktile, const uint8_t* vt, int lane, const v8i (&qop)[2],
                                           const v8i (&P)[2], float sig, SoftState& st, float (&d)[2], bool (&rose)[2],
                                           const v4f (&sh)[8][2], const float (&mh)[2], v4f (&sn)[8][2],
                                           v8i (&Pn)[2], float (&mn)[2], v4f (&O)[8][2], float (&rr)[2],
                                           bool rsel, const Copies& cp) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const v8i ones = {kOnes4, kOnes4, kOnes4, kOnes4, kOnes4, kOnes4, kOnes4, kOnes4};
  const uint8_t* kl = ktile + lane;   // lane = the lane's byte offset (16 * lane id)
  const uint8_t* vl = vt + lane;
  const float s8 = cast_scale(sig);
  const int se = st.se;
  v8i kop[2], vop[2];
  uint32_t vsc[2] = {0u, 0u};
  if (VF) {
    // the lane's 8 scale exponents (one per channel sub-tile), 8 bytes at 8*lane
    const uint2 s2 = *reinterpret_cast<const uint2*>(vt + kFp4CodeBytes + (lane >> 1));
    vsc[0] = s2.x;
    vsc[1] = s2.y;
  }
  vop[0] = ld_vop<VF>(vl, 0);
  vop[1] = ld_vop<VF>(vl, 1);
  uint32_t w[8][2];
  float mx[2] = {mh[0], mh[1]};
  // cast half i of the held scores: sub-tile i/4, query sub-tile (i/2)%2,
  // keys 2*(i%2) and 2*(i%2)+1 of the lane's four
  auto half = [&](int i) {
    const int t = i >> 2, q = (i >> 1) & 1, h = i & 1;
    if (h == 0) w[t][q] = 0;
    cast_half(sh[t][q], 2 * h, s8, st.cq[q], w[t][q]);
    if (h == 1) {
      Pn[q][t] = static_cast<int>(w[t][q]);
      asm volatile("" : "+v"(Pn[q][t]));
    } else {
      asm volatile("" : "+v"(w[t][q]));
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  // ---- first half: 18 slots ----
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    O[dt][0] = pv_mfma<VF, 0>(vop[dt & 1], P[0], O[dt][0], vsc, dt, se);
    asm volatile("" : "+v"(O[dt][0]));
    __builtin_amdgcn_sched_barrier(0);
    if (dt == 0) {
      // the held tile's last sub-tile, then the maximum after it
      max_acc(sh[7][0], mx[0]);
      rose[0] = new_max(st, 0, mx[0], sig, d[0]);
      asm volatile("" : "+v"(st.cq[0]), "+v"(d[0]));
    } else {
      half(2 * dt - 1);                    // slots 2, 4, .. 14: halves 1, 3, .. 13
    }
    __builtin_amdgcn_sched_barrier(0);
    O[dt][1] = pv_mfma<VF, 1>(vop[dt & 1], P[1], O[dt][1], vsc, dt, se);
    asm volatile("" : "+v"(O[dt][1]));
    __builtin_amdgcn_sched_barrier(0);
    if (dt == 0) {
      max_acc(sh[7][1], mx[1]);
      rose[1] = new_max(st, 1, mx[1], sig, d[1]);
      asm volatile("" : "+v"(st.cq[1]), "+v"(d[1]));
      half(0);
    } else {
      half(2 * dt);                        // slots 3, 5, .. 15: halves 2, 4, .. 14
    }
    if (dt + 2 < 8) vop[dt & 1] = ld_vop<VF>(vl, dt + 2);
    if (dt == 7) kop[0] = ld_op_lds_at(kl, 0);
    if ((dt & 1) && dt < 6) cp.issue(dt >> 1);      // parts 0, 1, 2
    __builtin_amdgcn_sched_barrier(0);
  }
  // row sums of tile kb
  v4f r0 = VF ? mfma_fp8_sb<0>(ones, P[0], zero, se) : mfma_fp8(ones, P[0], zero);
  asm volatile("" : "+v"(r0));
  __builtin_amdgcn_sched_barrier(0);
  half(15);
  half(16);
  kop[1] = ld_op_lds_at(kl, 1);
  __builtin_amdgcn_sched_barrier(0);
  v4f r1 = VF ? mfma_fp8_sb<1>(ones, P[1], zero, se) : mfma_fp8(ones, P[1], zero);
  asm volatile("" : "+v"(r1));
  __builtin_amdgcn_sched_barrier(0);
  half(17);
  half(18);
  __builtin_amdgcn_sched_barrier(0);
  // ---- second half: 16 slots ----
  mn[0] = mn[1] = kNegBig;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    sn[t][0] = mfma_fp8(kop[t & 1], qop[0], zero);
    __builtin_amdgcn_sched_barrier(0);
    if (t >= 1) {
      max_acc(sn[t - 1][0], mn[0]);
      asm volatile("" : "+v"(mn[0]));
    }
    if (2 * t < 13) half(19 + 2 * t);
    __builtin_amdgcn_sched_barrier(0);
    sn[t][1] = mfma_fp8(kop[t & 1], qop[1], zero);
    __builtin_amdgcn_sched_barrier(0);
    if (t >= 1) {
      max_acc(sn[t - 1][1], mn[1]);
      asm volatile("" : "+v"(mn[1]));
    }
    if (2 * t + 1 < 13) half(20 + 2 * t);
    if (t == 0) {
      // tile kb's row sums (ready two MFMAs after the second one): into l,
      // and into restore-weight slot rr where this lane group holds it
      st.l[0] += r0[0];
      st.l[1] += r1[0];
      if (rsel) {
        rr[0] = r0[0];
        rr[1] = r1[0];
      }
      asm volatile("" : "+v"(st.l[0]), "+v"(st.l[1]), "+v"(rr[0]), "+v"(rr[1]));
    }
    if (t + 2 < 8) kop[t & 1] = ld_op_lds_at(kl, t + 2);
    if ((t & 1) && t < 6) cp.issue(3 + (t >> 1));   // parts 3, 4, 5
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Score tile without restore (tile 0 in the prologue).
__device__ __forceinline__ void score_tile(const uint8_t* ktile, int lane, const v8i (&qop)[2], v4f (&sc)[8][2]) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const v8i kop = ld_op_lds(ktile, t, lane);
    sc[t][0] = mfma_fp8(kop, qop[0], zero);
    sc[t][1] = mfma_fp8(kop, qop[1], zero);
  }
}

// Mask the key slots whose permuted position in the tile is >= kval (a
// ragged last tile).  Lane group g of score sub-tile t holds slots 16t+4g+i;
// E4M3 workspaces store position j in slot j, MXFP4 workspaces position
// mx_pos_of_slot(slot) = 64(t/4) + 16g + 4(t%4) + i.
template <int VF>
__device__ __forceinline__ void mask_tile(v4f (&sc)[8][2], int g, int kval) {
  // compare the lane-independent part against kval minus the lane group's
  // part: no per-key registers
  const int kr = kval - (VF ? 16 : 4) * g;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((VF ? 64 * (t >> 2) + 4 * (t & 3) : 16 * t) + i >= kr) sc[t][0][i] = sc[t][1][i] = kNegBig;
}

// Integer running max and ExpCast codes of the first tile.
__device__ __forceinline__ void softmax_tile(const v4f (&sc)[8][2], float sigma, SoftState& st, v8i (&P)[2]) {
  const float s8 = cast_scale(sigma);
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    float mx = max4(sc[0][qi]);
#pragma unroll
    for (int t = 1; t < 8; ++t) mx = fmaxf(mx, max4(sc[t][qi]));
    mx = max_over_rows(mx);
    const float mn = fmaxf(st.M[qi], ceilf(mx * sigma));
    st.M[qi] = mn;
    st.cq[qi] = cast_const(mn);
    const float c = st.cq[qi];
#pragma unroll
    for (int t = 0; t < 8; ++t) P[qi][t] = static_cast<int>(expcast4(sc[t][qi], s8, c));
  }
}

// Loop-invariant inputs of one workgroup's tile loop.
struct TileCtx {
  __amdgpu_buffer_rsrc_t kr, vr, sr, mr;   // this head's K8 tiles, V8 tiles, K scales, restore operands
  const float* ks;          // this head's K block scales
  const uint8_t* muop;      // this head's restore operands
  uint8_t* grp0;            // LDS group buffers for the restore operands
  uint8_t* grp1;            // (even and odd groups)
  float sqs, sm_scale;
  int nblk, kval_last, tid, lane, g, l16, w;
  int lane16;   // 16 * lane, opaque to the compiler (kept in one register)
};

// Per-wave accumulators carried across tiles.
struct TileAcc {
  v4f O[8][2];     // O^T: lane holds channels 16dt+4g+i of query l16 (+16 per sub-tile)
  v8i P[2];        // E4M3 codes of the current tile (P^T operand)
  float rr[4][2];  // deferred restore weights: lane group g, slot j holds the
                   // row sum of tile 16G+4g+j of the current group G
  SoftState st;
  v4f sh[8][2];    // raw scores of the next tile (cast in the next step)
  float mh[2];     // their per-lane partial maxima
  float sig;       // their sigma (log2-domain score scale)
};

// The copies of one step: K(tk) with its scale into kfree, V(tv) into vfree,
// and restore-operand row `row` into its group buffer -- parts 1..kDmaPerTile
// K, then V (every wave), part 0 the scale and part 2*kDmaPerTile+1 the row
// (wave 0 only) -- issued one at a time at points spread over the step, so
// that the workgroup's copies do not all queue at once.
template <int VF>
struct StepCopies {
  const TileCtx& c;
  uint32_t koff, voff, soff, roff;   // koff, voff: wave-uniform (tile and wave), the lane's part is c.lane16
  uint8_t* kdst;
  uint8_t* vdst;
  uint8_t* rdst;
  __device__ __forceinline__ StepCopies(const TileCtx& ctx, int tk, int tv, int row, uint8_t* kfree, uint8_t* vfree)
      : c(ctx) {
    // 16 * tid = 1024 * w + 16 * lane: the wave's part goes with the tile
    // offset into the scalar offset, the lane's part is c.lane16 (tk, tv
    // <= the last tile, so every copy stays inside the resource)
    koff = static_cast<uint32_t>(tk) * kTileBytes + static_cast<uint32_t>(c.w) * 1024;
    voff = static_cast<uint32_t>(tv) * kTileBytes + static_cast<uint32_t>(c.w) * 1024;
    soff = static_cast<uint32_t>(tk) * 4;
    roff = static_cast<uint32_t>(row) * kMuOpRowBytes + static_cast<uint32_t>(c.lane16);
    kdst = kfree;
    vdst = vfree;
    rdst = ((row / kMuOpGroup) & 1 ? c.grp1 : c.grp0) + (row % kMuOpGroup) * kMuOpRowBytes;
  }
  __device__ __forceinline__ void issue(int part) const {
    const int w = c.w;
    if (part == 0) {
      if (w == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.sr, (__attribute__((address_space(3))) void*)(kdst + kTileBytes),
                                                 4, soff, 0, 0, 0);
    } else if (part <= kDmaPerTile) {
      const int j = part - 1;
      copy16_to_lds_s(c.kr, static_cast<uint32_t>(c.lane16), koff + j * (16 * kAttnThreads),
                      kdst + j * (16 * kAttnThreads) + w * 1024);
    } else if (part <= 2 * kDmaPerTile) {
      const int j = part - 1 - kDmaPerTile;
      if (j < VTile<VF>::kDma) {
        copy16_to_lds_s(c.vr, static_cast<uint32_t>(c.lane16), voff + j * (16 * kAttnThreads),
                        vdst + j * (16 * kAttnThreads) + w * 1024);
      } else if (VF && w == 1) {
        // MXFP4: the tile's 512 scale bytes (and 512 unused bytes of the slot)
        copy16_to_lds_s(c.vr, static_cast<uint32_t>(c.lane16), voff - static_cast<uint32_t>(w) * 1024 + kFp4CodeBytes,
                        vdst + kFp4CodeBytes);
      }
    } else {
      if (w == 0) copy16_to_lds(c.mr, roff, rdst);
    }
  }
  __device__ __forceinline__ void issue_all() const {
#pragma unroll
    for (int p = 0; p < 2 * kDmaPerTile + 2; ++p) issue(p);
  }
};

// The copies of one step of a key half (the short-launch kernel: waves
// 4h..4h+3 own half h and copy its tiles): K(tk) with its scale into kdst
// and, when vdst is set, V(tv) into vdst, all at once at the start of the
// step before the tiles' use.  (Spread over the step's first half as the
// whole-item kernel spreads its copies, they land later, the barrier waits
// longer, and the short launches ran 9-13% slower.)
template <int VF>
struct HalfCopies {
  const TileCtx& c;
  int tk, tv;
  uint8_t* kdst;
  uint8_t* vdst;
  static constexpr int kHalfThreads = kAttnThreads / 2;
  static constexpr int kK = kTileBytes / (16 * kHalfThreads);                          // K copies per wave
  static constexpr int kV = (VF ? kFp4CodeBytes : kTileBytes) / (16 * kHalfThreads);  // V code copies per wave
  __device__ __forceinline__ HalfCopies(const TileCtx& ctx, int k_tile, int v_tile, uint8_t* kd, uint8_t* vd)
      : c(ctx), tk(k_tile), tv(v_tile), kdst(kd), vdst(vd) {}
  static_assert(kK % 2 == 0, "K copies in two halves");
  __device__ __forceinline__ void issue_k(int j0, int j1) const {
    const int hw = c.w & 3;   // wave within the half
    const uint32_t koff = static_cast<uint32_t>(tk) * kTileBytes + static_cast<uint32_t>(hw) * 1024;
    if (j0 == 0 && hw == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.sr, (__attribute__((address_space(3))) void*)(kdst + kTileBytes), 4,
                                               static_cast<uint32_t>(tk) * 4, 0, 0, 0);
#pragma unroll
    for (int j = j0; j < j1; ++j)
      copy16_to_lds_s(c.kr, static_cast<uint32_t>(c.lane16), koff + j * (16 * kHalfThreads),
                      kdst + j * (16 * kHalfThreads) + hw * 1024);
  }
  __device__ __forceinline__ void issue_v() const {
    if (!vdst) return;
    const int hw = c.w & 3;
    const uint32_t voff = static_cast<uint32_t>(tv) * kTileBytes + static_cast<uint32_t>(hw) * 1024;
#pragma unroll
    for (int j = 0; j < kV; ++j)
      copy16_to_lds_s(c.vr, static_cast<uint32_t>(c.lane16), voff + j * (16 * kHalfThreads),
                      vdst + j * (16 * kHalfThreads) + hw * 1024);
    if (VF && hw == 1)   // MXFP4: the tile's 512 scale bytes (and 512 unused bytes of the slot)
      copy16_to_lds_s(c.vr, static_cast<uint32_t>(c.lane16), voff - 1024 + kFp4CodeBytes, vdst + kFp4CodeBytes);
  }
  __device__ __forceinline__ void issue_all() const {
    issue_k(0, kK);
    issue_v();
  }
};
// The MFMA phase's copy points do nothing in the halves mode (its copies go
// out at the start of the step).
struct NoCopies {
  __device__ __forceinline__ void issue(int) const {}
};

// Deferred block-mean restore of one group of 16 tiles:
// O^T[dt][qi] += A_dt . B_qi over the group's tiles, A = mu/s_v (bf16 high
// and low parts, 16 channels x 16 tiles), B = the row-sum weights (16 tiles
// x 16 queries) split the same way; hi*hi + hi*lo + lo*hi.  A comes from
// `ops` (lane-ordered rows, 8 bytes per lane).
__device__ __forceinline__ v4s bf16x4_hi_lo(const float (&x)[4], v4s& lo) {
  v4s hi;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h = f32_to_bf16_bits(x[j]);
    hi[j] = static_cast<short>(h);
    lo[j] = static_cast<short>(f32_to_bf16_bits(x[j] - __uint_as_float(h << 16)));
  }
  return hi;
}
// The B operands of the restore: the weights split into bf16 high and low
// parts.
__device__ __forceinline__ void restore_weights(const float (&rr)[4][2], v4s (&bh)[2], v4s (&bl)[2]) {
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const float x[4] = {rr[0][qi], rr[1][qi], rr[2][qi], rr[3][qi]};
    bh[qi] = bf16x4_hi_lo(x, bl[qi]);
  }
}
// Restore MFMAs for the channel sub-tiles dt0 .. dt0+ND-1 (A[i] for dt0+i).
template <int ND>
__device__ __forceinline__ void restore_mfma(const v4s (&A)[ND][2], int dt0, const v4s (&bh)[2], const v4s (&bl)[2],
                                             v4f (&O)[8][2]) {
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int qi = 0; qi < 2; ++qi)
      O[dt0 + i][qi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[i][0], bh[qi], O[dt0 + i][qi], 0, 0, 0);
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int qi = 0; qi < 2; ++qi)
      O[dt0 + i][qi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[i][0], bl[qi], O[dt0 + i][qi], 0, 0, 0);
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int qi = 0; qi < 2; ++qi)
      O[dt0 + i][qi] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A[i][1], bh[qi], O[dt0 + i][qi], 0, 0, 0);
}

// Restore operands of a group from its LDS buffer.  The buffer is filled by
// copies whose completion the step barriers establish, which the compiler's
// wait insertion cannot see through a runtime-selected buffer; the reads are
// therefore written as one asm block that waits for its own results.  The
// outputs are early-clobber: the first load's result must not land in the
// address register the later loads of the block still read.
__device__ __forceinline__ void restore_ops_lds(const uint8_t* grp, int lane16, int half, v4s (&A)[4][2]) {
  // rows 2*dt + h for dt = 4*half .. 4*half+3: 8 consecutive rows; 8 bytes
  // per lane (lane16 = 16 * lane)
  const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<size_t>((const __attribute__((address_space(3))) uint8_t*)grp)) +
                        half * 8 * kMuOpRowBytes + (static_cast<uint32_t>(lane16) >> 1);
  asm volatile(
      "ds_read_b64 %0, %8 offset:0\n\t"
      "ds_read_b64 %1, %8 offset:512\n\t"
      "ds_read_b64 %2, %8 offset:1024\n\t"
      "ds_read_b64 %3, %8 offset:1536\n\t"
      "ds_read_b64 %4, %8 offset:2048\n\t"
      "ds_read_b64 %5, %8 offset:2560\n\t"
      "ds_read_b64 %6, %8 offset:3072\n\t"
      "ds_read_b64 %7, %8 offset:3584\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(A[0][0]), "=&v"(A[0][1]), "=&v"(A[1][0]), "=&v"(A[1][1]), "=&v"(A[2][0]), "=&v"(A[2][1]), "=&v"(A[3][0]),
        "=&v"(A[3][1])
      : "v"(addr)
      : "memory");
}

// One tile step kb (J = kb mod 4): the MFMA phase (P.V and row sums of
// tile kb with V in vcur -- the row sums going into l and the deferred
// restore weights --, codes of tile kb+1 against the maximum after it,
// scores of tile kb+2 with K in kcur), the step barrier, the masking of a
// ragged score tile, and the rescale of O, l and the weights of a query
// sub-tile whose maximum tile kb+1 raised (MXFP4: only when the anchor
// moves).  After the last tile of a group of 16 the group's restore
// runs.  Copies run ahead: this step copies K(kb+5) into kfree, V(kb+3) into
// vfree and restore-operand row kb+3 (distinct LDS arrays, so the copies
// overlap the reads of this step and the next two), as its last
// vector-memory instructions (see step_barrier).  Everything after the
// barrier works in registers or on a restore-operand group copied at least
// three steps before and not refilled for another thirteen, so it needs no
// barrier of its own.  Tile indices past the last tile are clamped to it
// and a score tile past the end is masked out entirely, which leaves the
// state unchanged (no rise, codes 0): every step runs the same code.
//
// HALVES (the short-launch kernel, each half of the workgroup on its own key
// range with two-slot rings): K(kb+2) is in kcur and V(kb) in vcur; the step
// first copies K(kb+3) into kfree and V(kb+1) into vfree (the slots that
// held K(kb+1) and V(kb-1), or K(0) at step 0, all last read before the
// previous barrier), all at once, and
// its barrier waits for them; a group's restore operands are read from
// global memory, for every group that holds a real tile of the half, at the
// group's last step (a half shorter than the step count runs masked steps
// past its end, whose zero row sums would overwrite the weight slots of a
// partial last group before any restore after the loop; the step count, a
// multiple of 16 no smaller than either half, ends every such group).
template <int VF, int J, bool HALVES = false>
__device__ __forceinline__ void tile_step(const TileCtx& c, int kb, const uint8_t* kcur, uint8_t* kfree,
                                          const uint8_t* vcur, uint8_t* vfree, const v8i (&qop)[2], TileAcc& acc) {
  const int nblk = c.nblk, last = nblk - 1, g = c.lane16 >> 8;   // lane group, from the kept 16*lane
  const StepCopies<VF> cp(c, kb + kStages + 1 < last ? kb + kStages + 1 : last,
                          kb + kStages - 1 < last ? kb + kStages - 1 : last, kb + kStages - 1, kfree, vfree);
  static_assert(2 * kDmaPerTile + 2 == 6, "six copy parts, one per sub-tile");
  if constexpr (HALVES)
    HalfCopies<VF>(c, kb + 3 < last ? kb + 3 : last, kb + 1 < last ? kb + 1 : last, kfree, vfree).issue_all();
  v8i Pn[2];
  float d[2], ks_new;
  bool rose[2];
  {
    v4f sn[8][2];
    float mn[2];
    // tile kb's row sum goes to l and to the restore weight of tile kb%16
    // of its group, held by lane group (kb/4)%4 in slot J
    if constexpr (HALVES)
      mfma_phase<VF>(kcur, vcur, c.lane16, qop, acc.P, acc.sig, acc.st, d, rose, acc.sh, acc.mh, sn, Pn, mn, acc.O,
                     acc.rr[J], (c.lane16 >> 8) == ((kb >> 2) & 3), NoCopies{});
    else
      mfma_phase<VF>(kcur, vcur, c.lane16, qop, acc.P, acc.sig, acc.st, d, rose, acc.sh, acc.mh, sn, Pn, mn, acc.O,
                     acc.rr[J], (c.lane16 >> 8) == ((kb >> 2) & 3), cp);
    // K(kb+2)'s scale (replicated per lane after the tile), read before the
    // barrier: the next step refills this buffer.  Wave-uniform, so it is
    // kept in a scalar register.
    ks_new = __int_as_float(__builtin_amdgcn_readfirstlane(
        *reinterpret_cast<const int*>(kcur + kTileBytes + (c.lane16 >> 2))));
    if constexpr (HALVES) {
      // every copy of this step has landed (s_waitcnt vmcnt(0) lgkmcnt(0))
      __builtin_amdgcn_s_waitcnt(0x70);
      __builtin_amdgcn_s_barrier();
    } else {
      step_barrier<VF>();
    }
    if (__builtin_expect(kb + 3 >= nblk, 0)) {
      // tile kb+2 is the last tile (keys past S masked) or past it (all masked)
      mask_tile<VF>(sn, g, kb + 2 == last ? c.kval_last : 0);
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        mn[qi] = max4(sn[0][qi]);
#pragma unroll
        for (int t = 1; t < 8; ++t) mn[qi] = max_acc4(mn[qi], sn[t][qi]);
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) acc.sh[t][0] = sn[t][0], acc.sh[t][1] = sn[t][1];
    acc.mh[0] = mn[0];
    acc.mh[1] = mn[1];
  }
  acc.sig = ((c.sqs * ks_new) * c.sm_scale) * kLog2e;
  // the maximum rose by d from tile kb to tile kb+1
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    if (__builtin_expect(rose[qi], 0)) {
      float alpha;
      bool resc = true;
      if (VF == 0) {
        // codes and accumulators against M: rescale by 2^-d
        alpha = ldexpf(1.0f, -static_cast<int>(fminf(d[qi], 160.0f)));
      } else {
        // the anchor scale of the next codes, 127 + (M' - A); past the span
        // the anchor moves up to M' and the accumulators are rescaled by
        // 2^(A - M')
        const int e = static_cast<int>((acc.st.se >> (8 * qi)) & 0xFF) - 127 +
                      static_cast<int>(fminf(d[qi], 2.0f * kAnchorSpan));
        const bool far = e > kAnchorSpan;
        alpha = far ? ldexpf(1.0f, -e) : 1.0f;
        acc.st.se = (acc.st.se & ~(0xFF << (8 * qi))) | ((far ? 127 : 127 + e) << (8 * qi));
        resc = __any(far);
      }
      if (resc) {
        acc.st.l[qi] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc.O[dt][qi] *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc.rr[j][qi] *= alpha;
      }
    }
  }
  acc.P[0] = Pn[0];
  acc.P[1] = Pn[1];
  if ((kb & (kMuOpGroup - 1)) == kMuOpGroup - 1) {
    if constexpr (HALVES) {
      if (kb - (kMuOpGroup - 1) < nblk) {
        // rows 16G .. 16G+15 of this half's operands, 8 bytes per lane
        const uint8_t* rows = c.muop + static_cast<int64_t>(kb / kMuOpGroup) * kMuOpGroup * kMuOpRowBytes +
                              (c.lane16 >> 1);
        v4s bh[2], bl[2];
        restore_weights(acc.rr, bh, bl);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          v4s A[4][2];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
              A[i][hl] = *reinterpret_cast<const v4s*>(rows + (2 * (4 * half + i) + hl) * kMuOpRowBytes);
          restore_mfma<4>(A, 4 * half, bh, bl, acc.O);
        }
      }
    } else {
      // the group's operand rows were copied by steps kb-18 .. kb-3, which
      // the barrier of step kb-1 has made visible
      // in two halves of four channel sub-tiles (fewer live registers)
      const uint8_t* grp = (kb / kMuOpGroup) & 1 ? c.grp1 : c.grp0;
      v4s bh[2], bl[2];
      restore_weights(acc.rr, bh, bl);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        v4s A[4][2];
        restore_ops_lds(grp, c.lane16, half, A);
        restore_mfma<4>(A, 4 * half, bh, bl, acc.O);
      }
    }
  }
}

// LDS buffers of one workgroup (distinct arrays for the ring slots: a copy
// into one provably does not alias reads of another).
struct AttnLds {
  uint8_t *kbuf0, *kbuf1, *kbuf2, *kbuf3, *vbuf0, *vbuf1, *vbuf2, *vbuf3, *grp0, *grp1;
};

// One piece of a work item: the queries of (b,h) = bh's pair of query blocks
// qp against key tiles [kv0, kv1) (kv0 a multiple of 16, the whole range for
// a whole item); REPAIR: the repair tiles follow (whole items only).  part == nullptr: the item is whole and its bf16 output is
// written; otherwise the piece's unnormalised O, row sums and reference
// exponents go to the partial slot `part` for the merge kernel.
template <int VF, bool REPAIR>
__device__ __forceinline__ void attn_piece(const AttnArgs& a, int bh, int qp, int kv0, int kv1, float* part,
                                           const AttnLds& L) {
  uint8_t* const kbuf0 = L.kbuf0;
  uint8_t* const kbuf1 = L.kbuf1;
  uint8_t* const kbuf2 = L.kbuf2;
  uint8_t* const kbuf3 = L.kbuf3;
  uint8_t* const vbuf0 = L.vbuf0;
  uint8_t* const vbuf1 = L.vbuf1;
  uint8_t* const vbuf2 = L.vbuf2;
  uint8_t* const vbuf3 = L.vbuf3;
  uint8_t* const kring[kStages] = {kbuf0, kbuf1, kbuf2, kbuf3};
  uint8_t* const vring[kStages] = {vbuf0, vbuf1, vbuf2, vbuf3};
  const int nfull = a.nblk;                        // tiles of the head
  const int b = bh / a.H, h = bh - b * a.H;

  // wave index made provably wave-uniform (scalar branches on it).  The
  // thread id passes through an empty asm first, so that nothing derived
  // from it can be hoisted out of a loop over pieces and held across one.
  int tid_raw = threadIdx.x;
  asm volatile("" : "+v"(tid_raw));
  const int tid = tid_raw, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int S = a.S;
  // waves 0-3 own query block 2*qp, waves 4-7 block 2*qp+1 (a missing second
  // block of an odd count is computed on a copy of the first and not stored)
  const int qb = 2 * qp + (w >> 2);
  const bool q_valid = qb < nfull;
  const int qbl = q_valid ? qb : nfull - 1;
  const int nblk = kv1 - kv0;                     // tiles of this piece
  const int wq = w & 3;                           // 32-query slice within the block

  TileCtx c;
  // the piece's tiles seen as a head of nblk tiles: resources start at tile
  // kv0 (restore-operand rows too: kv0 is a multiple of the 16-block group);
  // nblk <= 2^17 (S <= 2^24), so a head's tiles span less than 4 GB
  c.kr = head_rsrc(a.k8 + (static_cast<int64_t>(bh) * nfull + kv0) * kTileBytes,
                   static_cast<uint32_t>(nblk) * kTileBytes);
  c.vr = head_rsrc(a.v8 + (static_cast<int64_t>(bh) * nfull + kv0) * kTileBytes,
                   static_cast<uint32_t>(nblk) * kTileBytes);
  const int nrows = muop_rows(nfull);
  c.muop = a.v_muop + (static_cast<int64_t>(bh) * nrows + kv0) * kMuOpRowBytes;
  c.mr = head_rsrc(c.muop, static_cast<uint32_t>(nrows - kv0) * kMuOpRowBytes);
  c.ks = a.k_scale + static_cast<int64_t>(bh) * nfull + kv0;
  c.sr = head_rsrc(c.ks, static_cast<uint32_t>(nblk) * 4);
  c.grp0 = L.grp0;
  c.grp1 = L.grp1;
  c.sqs = a.q_scale[static_cast<int64_t>(bh) * nfull + qbl];
  c.sm_scale = a.sm_scale;
  c.nblk = nblk;
  // real keys in the piece's last tile
  c.kval_last = kv1 == nfull ? S - (nfull - 1) * kBlock : kBlock;
  c.tid = tid;
  c.w = w;
  c.lane = lane;
  {
    int l16b = lane * 16;
    asm volatile("" : "+v"(l16b));
    c.lane16 = l16b;
  }
  c.g = g;
  c.l16 = l16;
  const float sqs = c.sqs;

  const uint8_t* qtile = a.q8 + (static_cast<int64_t>(bh) * nfull + qbl) * kTileBytes;
  v8i qop[2];
  qop[0] = ld_op_global(qtile, 2 * wq, lane);
  qop[1] = ld_op_global(qtile, 2 * wq + 1, lane);

  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};

  TileAcc acc;
  acc.st.M[0] = acc.st.M[1] = kNegBig;
  acc.st.l[0] = acc.st.l[1] = 0.0f;
  acc.st.se = 0x7F7F7F7F;   // the anchor starts at tile 0's maximum
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc.O[dt][0] = acc.O[dt][1] = zero;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc.rr[j][0] = acc.rr[j][1] = 0.0f;

  // ---- prologue: K(0..3) with scales, V(0..2) and restore-operand rows
  // 0..2 into LDS; scores and codes of tile 0, scores of tile 1; then K(4)
  // into the slot of K(0) ----
  const int last = nblk - 1;
#pragma unroll
  for (int j = 0; j + 1 < kStages; ++j)
    StepCopies<VF>(c, j < last ? j : last, j < last ? j : last, j, kring[j], vring[j]).issue_all();
  {
    const StepCopies<VF> cp(c, kStages - 1 < last ? kStages - 1 : last, 0, 0, kring[kStages - 1], vring[0]);
#pragma unroll
    for (int p = 0; p <= kDmaPerTile; ++p) cp.issue(p);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  {
    v4f sc[8][2];
    score_tile(kbuf0, lane, qop, sc);
    if (nblk == 1 && c.kval_last < kBlock) mask_tile<VF>(sc, g, c.kval_last);
    softmax_tile(sc, ((sqs * c.ks[0]) * a.sm_scale) * kLog2e, acc.st, acc.P);
  }
  // scores of tile 1 (a copy of tile 0, masked out, when there is none):
  // their codes are cast in the first step
  score_tile(kbuf1, lane, qop, acc.sh);
  if (nblk <= 2) mask_tile<VF>(acc.sh, g, nblk == 2 ? c.kval_last : 0);
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    acc.mh[qi] = max4(acc.sh[0][qi]);
#pragma unroll
    for (int t = 1; t < 8; ++t) acc.mh[qi] = max_acc4(acc.mh[qi], acc.sh[t][qi]);
  }
  acc.sig = ((sqs * c.ks[last < 1 ? last : 1]) * a.sm_scale) * kLog2e;
  __syncthreads();   // kring[0] and kring[1] are refilled from here on
  {
    const StepCopies<VF> cp(c, kStages < last ? kStages : last, 0, 0, kring[0], vring[0]);
#pragma unroll
    for (int p = 0; p <= kDmaPerTile; ++p) cp.issue(p);
  }

  // Step kb reads K(kb+2) from kring[(kb+2)%S] and V(kb) from vring[kb%S]
  // (S = kStages), and refills kring[(kb+1)%S] with K(kb+S+1) and
  // vring[(kb+S-1)%S] with V(kb+S-1).  The loop is unrolled S times so that
  // every buffer is a fixed array.
  static_assert(kStages == 4, "tile_step<J> takes J = kb mod 4");
  int kb = 0;
  for (; kb + kStages <= nblk; kb += kStages) {
    tile_step<VF, 0>(c, kb, kbuf2, kbuf1, vbuf0, vbuf3, qop, acc);
    tile_step<VF, 1>(c, kb + 1, kbuf3, kbuf2, vbuf1, vbuf0, qop, acc);
    tile_step<VF, 2>(c, kb + 2, kbuf0, kbuf3, vbuf2, vbuf1, qop, acc);
    tile_step<VF, 3>(c, kb + 3, kbuf1, kbuf0, vbuf3, vbuf2, qop, acc);
  }
  if (kb < nblk) tile_step<VF, 0>(c, kb, kbuf2, kbuf1, vbuf0, vbuf3, qop, acc);
  if (kb + 1 < nblk) tile_step<VF, 1>(c, kb + 1, kbuf3, kbuf2, vbuf1, vbuf0, qop, acc);
  if (kb + 2 < nblk) tile_step<VF, 2>(c, kb + 2, kbuf0, kbuf3, vbuf2, vbuf1, qop, acc);
  // drain the copies still in flight before the workgroup retires
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // the lane's index values again, from the one register the tile loop kept
  // (16 * lane), instead of keeping the originals live across it
  const int lane_p = c.lane16 >> 4, g_p = lane_p >> 4, l16_p = lane_p & 15;

  // restore of the last, partial group (its operand rows may not all have
  // been copied; read them from global memory).  Weight slots of tiles past
  // the last hold stale sums but meet zero operands.
  if ((last & (kMuOpGroup - 1)) != kMuOpGroup - 1) {
    const uint8_t* rows = c.muop + static_cast<int64_t>(last / kMuOpGroup) * kMuOpGroup * kMuOpRowBytes + lane_p * 8;
    v4s A[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) A[dt][hl] = *reinterpret_cast<const v4s*>(rows + (2 * dt + hl) * kMuOpRowBytes);
    v4s bh[2], bl[2];
    restore_weights(acc.rr, bh, bl);
    restore_mfma<8>(A, 0, bh, bl, acc.O);
  }

  SoftState& st = acc.st;
  v4f (&O)[8][2] = acc.O;
  const vc_head_hdr hd = a.hdr[bh];

  // ---- residual repair tiles (codes against the final maximum) ----
  if (REPAIR && a.nrep_pad > 0) {
    const int nrep = hd.nrep;
    const float fe = hd.rep_scale / hd.v_scale;
    const uint8_t* rk = a.rep_k8 + static_cast<int64_t>(bh) * a.nrep_pad * kD;
    const uint8_t* re = a.rep_e8 + static_cast<int64_t>(bh) * a.nrep_pad * kD;
    const float* rks = a.rep_ks + static_cast<int64_t>(bh) * a.nrep_pad;
    for (int rt = 0; rt < a.nrep_pad / kBlock; ++rt) {
      v8i Pr[2];
      // the tile's K operands and key scales are loaded together (one round
      // trip from global memory rather than one per sub-tile)
      v8i kops[8];
      float4 ksc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        kops[t] = ld_op_global(rk + static_cast<int64_t>(rt) * kTileBytes, t, lane_p);
        ksc[t] = *reinterpret_cast<const float4*>(rks + rt * kBlock + 16 * t + 4 * g_p);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const v8i kop = kops[t];
        const float kst[4] = {ksc[t].x, ksc[t].y, ksc[t].z, ksc[t].w};
        const v4f s0 = mfma_fp8(kop, qop[0], zero);
        const v4f s1 = mfma_fp8(kop, qop[1], zero);
        uint32_t w0 = 0, w1 = 0;
        // slots past the repair set cast to code 0
#ifndef VC_ABLATION_EXP_CAST
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = rt * kBlock + 16 * t + 4 * g_p + i;
          const float sig = ((sqs * kst[i]) * a.sm_scale) * kLog2e;
          // (the ExpCast constants written out: as calls of cast_scale and
          // cast_const the register allocation of the whole kernel spills)
          const float s8j = j < nrep ? 8.0f * sig : 0.0f;
          const float c0 = j < nrep ? 120.0f - 8.0f * st.M[0] : -1.0f;
          const float c1 = j < nrep ? 120.0f - 8.0f * st.M[1] : -1.0f;
          w0 = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s0[i], s8j, c0), i, w0);
          w1 = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(s1[i], s8j, c1), i, w1);
        }
#else
        // pairs of keys: two exponentials and one packed conversion each
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          float sa[2], b0[2], b1[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int j = rt * kBlock + 16 * t + 4 * g_p + i + k;
            const float sig = ((sqs * kst[i + k]) * a.sm_scale) * kLog2e;
            sa[k] = j < nrep ? cast_scale(sig) : 0.0f;
            b0[k] = j < nrep ? cast_const(st.M[0]) : kCastOff;
            b1[k] = j < nrep ? cast_const(st.M[1]) : kCastOff;
          }
          w0 = pcast2v(s0[i], s0[i + 1], sa, b0, i >> 1, w0);
          w1 = pcast2v(s1[i], s1[i + 1], sa, b1, i >> 1, w1);
        }
#endif
        Pr[0][t] = static_cast<int>(w0);
        Pr[1][t] = static_cast<int>(w1);
      }
      // likewise the tile's eight error operands
      v8i eops[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) eops[dt] = ld_op_global(re + static_cast<int64_t>(rt) * kTileBytes, dt, lane_p);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v8i eop = eops[dt];
        // codes against M, accumulators against the anchor
        const v4f o0 = mfma_fp8_sb<0>(eop, Pr[0], zero, st.se);
        const v4f o1 = mfma_fp8_sb<1>(eop, Pr[1], zero, st.se);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          O[dt][0][i] = fmaf(fe, o0[i], O[dt][0][i]);
          O[dt][1][i] = fmaf(fe, o1[i], O[dt][1][i]);
        }
      }
    }
  }

  if (part) {
    // ---- a piece: unnormalised O, row sums and the exponent they are
    // relative to (M, or the MXFP4 anchor A = M - (se byte - 127)) ----
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      const int r = (w >> 2) * kBlock + 16 * (2 * wq + qi) + l16_p;   // query row within the pair
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<v4f*>(part + r * kD + 16 * dt + 4 * g_p) = O[dt][qi];
      if (g_p == 0) {
        part[256 * kD + r] = st.l[qi];
        part[256 * kD + 256 + r] = st.M[qi] - static_cast<float>(static_cast<int>((st.se >> (8 * qi)) & 0xFF) - 127);
      }
    }
    return;
  }
  // ---- epilogue: out = bf16(s_v * O / l), original query order ----
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int q = qb * kBlock + 16 * (2 * wq + qi) + l16_p;
    if (q_valid && q < S) {
      const float f = hd.v_scale / st.l[qi];
      uint16_t* orow = a.out + b * a.osB + static_cast<int64_t>(q) * a.osS + h * a.osH;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint32_t lo = f32_to_bf16_bits(O[dt][qi][0] * f) | (f32_to_bf16_bits(O[dt][qi][1] * f) << 16);
        const uint32_t hi = f32_to_bf16_bits(O[dt][qi][2] * f) | (f32_to_bf16_bits(O[dt][qi][3] * f) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g_p) = make_uint2(lo, hi);
      }
    }
  }
}

// Workgroup id -> work index, XCD-aware: the hardware deals workgroup ids
// round-robin over the 8 XCDs; XCD x gets a contiguous range of the `total`
// work indices (consecutive query blocks of one head share its L2).
__device__ __forceinline__ int xcd_order(int total, int wg) {
  const int xcd = wg & 7, idx = wg >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

#define VC_ATTN_LDS_DECL(VF)                                                       \
  static_assert(kStages == 4, "buffer declarations below");                         \
  __shared__ __align__(16) uint8_t kbuf0[kKBufBytes]; /* K codes + tile scale */    \
  __shared__ __align__(16) uint8_t kbuf1[kKBufBytes];                               \
  __shared__ __align__(16) uint8_t kbuf2[kKBufBytes];                               \
  __shared__ __align__(16) uint8_t kbuf3[kKBufBytes];                               \
  __shared__ __align__(16) uint8_t vbuf0[VTile<VF>::kBytes];                        \
  __shared__ __align__(16) uint8_t vbuf1[VTile<VF>::kBytes];                        \
  __shared__ __align__(16) uint8_t vbuf2[VTile<VF>::kBytes];                        \
  __shared__ __align__(16) uint8_t vbuf3[VTile<VF>::kBytes];                        \
  __shared__ __align__(16) uint8_t grp0[kGrpBytes]; /* restore operands, even */    \
  __shared__ __align__(16) uint8_t grp1[kGrpBytes]; /* and odd groups */            \
  const AttnLds L = {kbuf0, kbuf1, kbuf2, kbuf3, vbuf0, vbuf1, vbuf2, vbuf3, grp0, grp1}

// Whole work items: (b,h) and query-block pair, in XCD-aware order.  REPAIR:
// the workspace has a repair set (the repair tiles follow the main loop);
// without one the kernel is built without that code.
template <int VF, bool REPAIR>
__global__ void __launch_bounds__(kAttnThreads, 1) k_vc_attn_fwd(AttnArgs a) {
  VC_ATTN_LDS_DECL(VF);
  const int npair = (a.nblk + 1) >> 1;
  const int item = xcd_order(a.whole, blockIdx.x);
  attn_piece<VF, REPAIR>(a, item / npair, item - (item / npair) * npair, 0, a.nblk, nullptr, L);
}

// The cut items, launched after the whole ones: workgroup t runs groups
// [t*per, t*per + per) of the cut items' (item, 16-tile group) sequence, as
// one or two pieces (the run crosses at most one item boundary); a piece that
// is a whole item writes its output directly.
struct AttnTailArgs {
  AttnArgs a;
  AttnTail tl;
};
template <int VF>
__global__ void __launch_bounds__(kAttnThreads, 1) k_vc_attn_tail(AttnTailArgs args) {
  VC_ATTN_LDS_DECL(VF);
  const AttnArgs& a = args.a;
  const AttnTail& tl = args.tl;
  const int npair = (a.nblk + 1) >> 1, ngrp = tl.ngrp;
  const int t = xcd_order(tl.tail_wg, blockIdx.x);
  int g = t * tl.per;
  const int gend = min(g + tl.per, tl.tail * ngrp);
#pragma nounroll
  for (int j = 0; j < 2 && g < gend; ++j) {
    const int i = g / ngrp, g0 = g - i * ngrp, g1 = min(ngrp, g0 + (gend - g));
    const int item = a.whole + i;
    float* part = g0 == 0 && g1 == ngrp ? nullptr : tl.part + static_cast<int64_t>(2 * t + j) * kPartFloats;
    if (j) __syncthreads();   // every wave is done with the previous piece's LDS
    // (no repair tiles: workspaces with a repair set are never cut)
    attn_piece<VF, false>(a, item / npair, item - (item / npair) * npair, kAttnGroup * g0,
                          min(a.nblk, kAttnGroup * g1), part, L);
    g += g1 - g0;
  }
}

// Merge of the pieces of a cut item (grid: cut items x 8 blocks of 32 query
// rows; 256 threads): with e_i the pieces' reference exponents, E = max e_i
// and w_i = 2^(e_i - E), out = bf16(s_v * sum_i w_i O_i / sum_i w_i l_i).
// Every factor is a power of two, so this is the online softmax's own
// rescale.  Thread t moves 16 B of 4 rows (lanes t%32 cover a row's 128
// channels); all its loads of one pass are independent.
constexpr int kMergeRowBlocks = 8;
__global__ void __launch_bounds__(256) k_vc_attn_merge(AttnArgs a, AttnTail tl) {
  const int i = blockIdx.x, ngrp = tl.ngrp, per = tl.per;
  const int wf = (i * ngrp) / per, wl = ((i + 1) * ngrp - 1) / per;
  if (wf == wl) return;                     // the item ran whole in one workgroup
  const int item = a.whole + i;
  const int npair = (a.nblk + 1) >> 1;
  const int bh = item / npair, qp = item - bh * npair;
  const int b = bh / a.H, h = bh - b * a.H;
  const float sv = a.hdr[bh].v_scale;
  const int c4 = threadIdx.x & 31;
  const int r0 = blockIdx.y * (256 / kMergeRowBlocks) + (threadIdx.x >> 5);
  // slot of workgroup wv's piece of item i: its first piece if its run starts inside the item
  auto slot = [&](int wv) {
    return tl.part + static_cast<int64_t>(2 * wv + (wv * per >= i * ngrp ? 0 : 1)) * kPartFloats;
  };
  constexpr int kRows = 256 / kMergeRowBlocks / 8;
  float e[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) e[k] = -3.0e38f;
  for (int wv = wf; wv <= wl; ++wv) {
    const float* p = slot(wv) + 256 * kD + 256;
#pragma unroll
    for (int k = 0; k < kRows; ++k) e[k] = fmaxf(e[k], p[r0 + 8 * k]);
  }
  float l[kRows];
  v4f o[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    l[k] = 0.0f;
    o[k] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  for (int wv = wf; wv <= wl; ++wv) {
    const float* p = slot(wv);
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int r = r0 + 8 * k;
      const float sc = ldexpf(1.0f, static_cast<int>(fmaxf(p[256 * kD + 256 + r] - e[k], -200.0f)));
      l[k] += sc * p[256 * kD + r];
      o[k] += sc * *reinterpret_cast<const v4f*>(p + r * kD + 4 * c4);
    }
  }
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int q = qp * 256 + r0 + 8 * k;
    if (q < a.S) {
      const float f = sv / l[k];
      const uint32_t lo = f32_to_bf16_bits(o[k][0] * f) | (f32_to_bf16_bits(o[k][1] * f) << 16);
      const uint32_t hi = f32_to_bf16_bits(o[k][2] * f) | (f32_to_bf16_bits(o[k][3] * f) << 16);
      *reinterpret_cast<uint2*>(a.out + b * a.osB + static_cast<int64_t>(q) * a.osS + h * a.osH + 4 * c4) =
          make_uint2(lo, hi);
    }
  }
}

// Short launches (no more query blocks than compute units, attn_split's
// `halves`): one workgroup per (b,h) and 128-query block qb.  Waves 0-3 take
// key tiles [0, ka) and waves 4-7 tiles [ka, nblk), ka = 16 * ceil(ngrp/2),
// each wave owning the same 32 queries (w % 4) of qb in both halves, so the
// per-wave work of a step is that of the whole-item kernel.  Each half
// streams its tiles through its own four slots, a two-slot K ring and a
// two-slot V ring (the prologue fills all four at once); both halves run
// ka steps (the shorter one masked past its end) under one barrier per step.
// Then each wave and its partner in the other half swap half of O, and l
// and their reference exponents, through LDS, and each adds the partner's
// part to its own with the weights 2^(e_i - max e) -- the merge of the cut
// items, inside the workgroup -- and writes its 64 output channels.
struct HalfLds {
  uint8_t *k0, *k1, *k2, *k3, *v0, *v1, *v2, *v3;
  uint8_t* junk;      // 8 waves x 256 bytes: landing room of the L2 warm-up
};
template <int VF>
__device__ __forceinline__ void attn_halves(const AttnArgs& a, int bh, int qb, int ka, const HalfLds& L) {
  const int nfull = a.nblk;
  const int b = bh / a.H, h = bh - b * a.H;
  int tid_raw = threadIdx.x;
  asm volatile("" : "+v"(tid_raw));
  const int tid = tid_raw, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int S = a.S;
  const int half = w >> 2, wq = w & 3;
  const int kv0 = half ? ka : 0, kv1 = half ? nfull : (ka < nfull ? ka : nfull);
  const int nblk = kv1 - kv0;           // this half's tiles (>= 1)
  uint8_t* const k0 = half ? L.k2 : L.k0;
  uint8_t* const k1 = half ? L.k3 : L.k1;
  uint8_t* const v0 = half ? L.v2 : L.v0;
  uint8_t* const v1 = half ? L.v3 : L.v1;

  // L2 warm-up.  The head's nfull workgroups (one per query block, placed on
  // one XCD by xcd_order where the head's blocks fill it) each touch one
  // 128-byte line per lane: K tile qb (waves 0-1), V tile qb (waves 2-3)
  // and every nfull-th line of the restore operands (waves 4-7), so the
  // head's tiles come into L2 at once, at the start, and the copies of the
  // steps find them there instead of each missing in turn.  The four bytes
  // a lane fetches land in a buffer of their own that no one reads.
  {
    const uint32_t line = static_cast<uint32_t>(tid & 127) * 128;
    uint8_t* const junk = L.junk + w * 256;
    if (w < 4) {
      const uint8_t* const base = (w < 2 ? a.k8 : a.v8) + static_cast<int64_t>(bh) * nfull * kTileBytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(head_rsrc(base, static_cast<uint32_t>(nfull) * kTileBytes),
                                               (__attribute__((address_space(3))) void*)junk, 4,
                                               static_cast<uint32_t>(qb) * kTileBytes + line, 0, 0, 0);
    } else {
      const int nrows_h = muop_rows(nfull);
      const uint8_t* const base = a.v_muop + static_cast<int64_t>(bh) * nrows_h * kMuOpRowBytes;
      const uint32_t l = static_cast<uint32_t>(tid - 256) * static_cast<uint32_t>(nfull) + static_cast<uint32_t>(qb);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(head_rsrc(base, static_cast<uint32_t>(nrows_h) * kMuOpRowBytes),
                                               (__attribute__((address_space(3))) void*)junk, 4, l * 128, 0, 0, 0);
    }
  }

  TileCtx c;
  c.kr = head_rsrc(a.k8 + (static_cast<int64_t>(bh) * nfull + kv0) * kTileBytes,
                   static_cast<uint32_t>(nblk) * kTileBytes);
  c.vr = head_rsrc(a.v8 + (static_cast<int64_t>(bh) * nfull + kv0) * kTileBytes,
                   static_cast<uint32_t>(nblk) * kTileBytes);
  const int nrows = muop_rows(nfull);
  c.muop = a.v_muop + (static_cast<int64_t>(bh) * nrows + kv0) * kMuOpRowBytes;
  c.mr = head_rsrc(c.muop, static_cast<uint32_t>(nrows - kv0) * kMuOpRowBytes);
  c.ks = a.k_scale + static_cast<int64_t>(bh) * nfull + kv0;
  c.sr = head_rsrc(c.ks, static_cast<uint32_t>(nblk) * 4);
  c.grp0 = nullptr;
  c.grp1 = nullptr;
  c.sqs = a.q_scale[static_cast<int64_t>(bh) * nfull + qb];
  c.sm_scale = a.sm_scale;
  c.nblk = nblk;
  c.kval_last = kv1 == nfull ? S - (nfull - 1) * kBlock : kBlock;
  c.tid = tid;
  c.w = w;
  c.lane = lane;
  {
    int l16b = lane * 16;
    asm volatile("" : "+v"(l16b));
    c.lane16 = l16b;
  }
  c.g = g;
  c.l16 = l16;
  const float sqs = c.sqs;
  const uint8_t* qtile = a.q8 + (static_cast<int64_t>(bh) * nfull + qb) * kTileBytes;
  v8i qop[2];
  qop[0] = ld_op_global(qtile, 2 * wq, lane);
  qop[1] = ld_op_global(qtile, 2 * wq + 1, lane);
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  TileAcc acc;
  acc.st.M[0] = acc.st.M[1] = kNegBig;
  acc.st.l[0] = acc.st.l[1] = 0.0f;
  acc.st.se = 0x7F7F7F7F;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc.O[dt][0] = acc.O[dt][1] = zero;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc.rr[j][0] = acc.rr[j][1] = 0.0f;

  // ---- prologue: K(0) into k0, V(0) into v0, K(1) into k1 and K(2) into
  // v1, all at once; scores and codes of tile 0, scores of tile 1 ----
  const int last = nblk - 1;
  HalfCopies<VF>(c, 0, 0, k0, v0).issue_all();
  HalfCopies<VF>(c, last < 1 ? last : 1, 0, k1, nullptr).issue_all();
  HalfCopies<VF>(c, last < 2 ? last : 2, 0, v1, nullptr).issue_all();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  {
    v4f sc[8][2];
    score_tile(k0, lane, qop, sc);
    if (nblk == 1 && c.kval_last < kBlock) mask_tile<VF>(sc, g, c.kval_last);
    softmax_tile(sc, ((sqs * c.ks[0]) * a.sm_scale) * kLog2e, acc.st, acc.P);
  }
  score_tile(k1, lane, qop, acc.sh);
  if (nblk <= 2) mask_tile<VF>(acc.sh, g, nblk == 2 ? c.kval_last : 0);
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    acc.mh[qi] = max4(acc.sh[0][qi]);
#pragma unroll
    for (int t = 1; t < 8; ++t) acc.mh[qi] = max_acc4(acc.mh[qi], acc.sh[t][qi]);
  }
  acc.sig = ((sqs * c.ks[last < 1 ? last : 1]) * a.sm_scale) * kLog2e;
  __syncthreads();   // k0 and k1 are refilled by step 0

  // The four slots are two rings: K(kb+2) is in v1 for even kb and in k1
  // for odd kb, V(kb) in v0 for even kb and in k0 for odd kb (step 0 puts
  // V(1) where K(0) was).  ka is a multiple of 16, so the loop has no
  // remainder.
  for (int kb = 0; kb < ka; kb += 4) {
    tile_step<VF, 0, true>(c, kb, v1, k1, v0, k0, qop, acc);
    tile_step<VF, 1, true>(c, kb + 1, k1, v1, k0, v0, qop, acc);
    tile_step<VF, 2, true>(c, kb + 2, v1, k1, v0, k0, qop, acc);
    tile_step<VF, 3, true>(c, kb + 3, k1, v1, k0, v0, qop, acc);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const int lane_p = c.lane16 >> 4, g_p = lane_p >> 4, l16_p = lane_p & 15;
  // (every group's restore ran in the loop, a partial last group's too:
  // its blocks past the head's end have zero operands and zero weights)

  // ---- the two halves meet in LDS (every wave is done with the slots) ----
  __syncthreads();
  float e[2];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi)
    e[qi] = acc.st.M[qi] - static_cast<float>(static_cast<int>((acc.st.se >> (8 * qi)) & 0xFF) - 127);
  // Each wave and its partner (w ^ 4, the same queries in the other half)
  // merge and write half of the channel sub-tiles: half 0 dt 0-3, half 1
  // dt 4-7.  Each leaves the other's four, lane-interleaved, in K buffer
  // wq (dt 0-3 in its first 8 KB, dt 4-7 in the second) and its l [2][16]
  // and e [2][16] in V buffer 0 (64 floats per half and wave).
  float* const xo = reinterpret_cast<float*>(wq == 0 ? L.k0 : wq == 1 ? L.k1 : wq == 2 ? L.k2 : L.k3);
  float* const xl = reinterpret_cast<float*>(L.v0) + wq * 128;
  // (the sub-tile indices are constants in each branch: O stays in registers)
  const auto send = [&](auto ds) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int qi = 0; qi < 2; ++qi)
        *reinterpret_cast<v4f*>(xo + (((ds + i) * 2 + qi) * 64 + lane_p) * 4) = acc.O[ds + i][qi];
  };
  if (half)
    send(std::integral_constant<int, 0>{});
  else
    send(std::integral_constant<int, 4>{});
  if (g_p == 0) {
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      xl[half * 64 + qi * 16 + l16_p] = acc.st.l[qi];
      xl[half * 64 + 32 + qi * 16 + l16_p] = e[qi];
    }
  }
  __syncthreads();
  const float sv = a.hdr[bh].v_scale;
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    // (l, e) of half 0 and of half 1; the weights 2^(e_i - max e)
    const float lp = xl[(1 - half) * 64 + qi * 16 + l16_p], ep = xl[(1 - half) * 64 + 32 + qi * 16 + l16_p];
    const float la = half ? lp : acc.st.l[qi], ea = half ? ep : e[qi];
    const float lb = half ? acc.st.l[qi] : lp, eb = half ? e[qi] : ep;
    const float E = fmaxf(ea, eb);
    const float wa = ldexpf(1.0f, static_cast<int>(fmaxf(ea - E, -200.0f)));
    const float wb = ldexpf(1.0f, static_cast<int>(fmaxf(eb - E, -200.0f)));
    const float f = sv / (wa * la + wb * lb);
    const int q = qb * kBlock + 16 * (2 * wq + qi) + l16_p;
    if (q < S) {
      uint16_t* orow = a.out + b * a.osB + static_cast<int64_t>(q) * a.osS + h * a.osH;
      const auto write = [&](auto d0, auto mine_b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dt = d0 + i;
          const v4f op = *reinterpret_cast<const v4f*>(xo + ((dt * 2 + qi) * 64 + lane_p) * 4);
          const v4f o = mine_b ? wa * op + wb * acc.O[dt][qi] : wa * acc.O[dt][qi] + wb * op;
          const uint32_t lo = f32_to_bf16_bits(o[0] * f) | (f32_to_bf16_bits(o[1] * f) << 16);
          const uint32_t hi = f32_to_bf16_bits(o[2] * f) | (f32_to_bf16_bits(o[3] * f) << 16);
          *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * g_p) = make_uint2(lo, hi);
        }
      };
      if (half)
        write(std::integral_constant<int, 4>{}, std::true_type{});
      else
        write(std::integral_constant<int, 0>{}, std::false_type{});
    }
  }
}

template <int VF>
__global__ void __launch_bounds__(kAttnThreads, 1) k_vc_attn_halves(AttnArgs a, int ka) {
  static_assert(kStages == 4, "four K and four V buffers, two of each per half");
  __shared__ __align__(16) uint8_t kbuf0[kKBufBytes];
  __shared__ __align__(16) uint8_t kbuf1[kKBufBytes];
  __shared__ __align__(16) uint8_t kbuf2[kKBufBytes];
  __shared__ __align__(16) uint8_t kbuf3[kKBufBytes];
  // (every slot takes K and V tiles in turn, so all are K-sized)
  __shared__ __align__(16) uint8_t vbuf0[kKBufBytes];
  __shared__ __align__(16) uint8_t vbuf1[kKBufBytes];
  __shared__ __align__(16) uint8_t vbuf2[kKBufBytes];
  __shared__ __align__(16) uint8_t vbuf3[kKBufBytes];
  __shared__ __align__(16) uint8_t junk[kAttnWaves * 256];
  const HalfLds L = {kbuf0, kbuf1, kbuf2, kbuf3, vbuf0, vbuf1, vbuf2, vbuf3, junk};
  const int nq = a.nblk;
  const int item = xcd_order(gridDim.x, blockIdx.x);
  const int bh = item / nq;
  attn_halves<VF>(a, bh, item - bh * nq, ka, L);
}

hipError_t launch_attention(const AttnArgs& a, const AttnTail& tl, hipStream_t st) {
  const bool fp4 = a.v_format == VC_V_MXFP4;
  if (tl.halves > 0) {
    // one workgroup per (b,h) and query block
    if (fp4)
      hipLaunchKernelGGL(k_vc_attn_halves<VC_V_MXFP4>, dim3(tl.halves), dim3(kAttnThreads), 0, st, a, tl.ka);
    else
      hipLaunchKernelGGL(k_vc_attn_halves<VC_V_E4M3>, dim3(tl.halves), dim3(kAttnThreads), 0, st, a, tl.ka);
    return hipGetLastError();
  }
  if (a.whole > 0) {
    // (MXFP4 workspaces have no repair set)
    if (fp4)
      hipLaunchKernelGGL((k_vc_attn_fwd<VC_V_MXFP4, false>), dim3(a.whole), dim3(kAttnThreads), 0, st, a);
    else if (a.nrep_pad > 0)
      hipLaunchKernelGGL((k_vc_attn_fwd<VC_V_E4M3, true>), dim3(a.whole), dim3(kAttnThreads), 0, st, a);
    else
      hipLaunchKernelGGL((k_vc_attn_fwd<VC_V_E4M3, false>), dim3(a.whole), dim3(kAttnThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tl.tail == 0) return hipSuccess;
  const AttnTailArgs ta = {a, tl};
  if (fp4)
    hipLaunchKernelGGL(k_vc_attn_tail<VC_V_MXFP4>, dim3(tl.tail_wg), dim3(kAttnThreads), 0, st, ta);
  else
    hipLaunchKernelGGL(k_vc_attn_tail<VC_V_E4M3>, dim3(tl.tail_wg), dim3(kAttnThreads), 0, st, ta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_vc_attn_merge, dim3(tl.tail, kMergeRowBlocks), dim3(256), 0, st, a, tl);
  return hipGetLastError();
}

}  // namespace vc

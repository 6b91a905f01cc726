// vc_common.hpp -- device helpers shared by the VC-Attention kernels (gfx950).
//
// E4M3 here is the OCP E4M3FN format that gfx950's FP8 MFMA consumes
// (cbsz/blgp = 0): sign, 4 exponent bits (bias 7), 3 mantissa bits, no
// infinities, 0x7F/0xFF NaN, largest finite 448 (0x7E).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "vc.h"

namespace vc {

constexpr int kD = 128;          // head dimension
constexpr int kBlock = 128;      // tokens per quantisation block / KV tile
constexpr int kTileBytes = kBlock * kD;
constexpr int kMaxK = 64;        // clusters per head
// Block-mean restore operands (v_muop): per head, rows of 512 bytes; group
// G = 16 consecutive blocks; row 16G + 2*dt + h holds the A operand of a
// 16x16x16 bf16 MFMA for channels 16dt..16dt+15 and blocks 16G..16G+15 --
// lane l's 8 bytes are 4 bf16 values for channel 16dt + l%16 and blocks
// 16G + 4*(l/16) + j, j = 0..3 -- of the high (h = 0) or low (h = 1) bf16
// part of mu_b/s_v.  Blocks past the last are zero; a head has
// muop_rows(nblk) rows (room for the attention kernel to read three rows
// past the last block).
constexpr int kMuOpRowBytes = 512;
constexpr int kMuOpGroup = 16;
__host__ __device__ inline int muop_rows(int nblk) { return kMuOpGroup * ((nblk + 3 + kMuOpGroup - 1) / kMuOpGroup); }
// Tokens per k-means assignment / sort chunk (one workgroup each): 1024,
// halved down to 128 while the B*H*chunks grid would not fill the GPU
// several times over (short sequences).
constexpr int kAsgTokMax = 1024;
constexpr int kAsgTokMin = 128;
__host__ __device__ inline int asg_tokens(int64_t BH, int S) {
  int t = kAsgTokMax;
  while (t > kAsgTokMin && BH * ((S + t - 1) / t) < 1024) t >>= 1;
  return t;
}

// Work split of one attention launch.  A work item is one (b,h) and pair of
// 128-query blocks; one workgroup holds a compute unit (its LDS), so a launch
// runs in rounds of kAttnSlots items.  With items = q*kAttnSlots + R, the
// first q*kAttnSlots items run whole, and the last R (0 < R < kAttnSlots,
// the partial last round -- or all items when there are fewer than
// kAttnSlots) are cut along the key axis into runs of 16-tile groups
// (ngrp = ceil(nblk/16) per item) spread evenly over tail_wg <= kAttnSlots
// workgroups of `per` groups each, so that the last round takes about R/kAttnSlots
// of a whole item's time instead of all of it.  A workgroup's run crosses at
// most one item boundary (per < ngrp), so it holds at most two pieces; a piece
// that is not a whole item leaves its unnormalised O, row sum and reference
// exponent in a partial slot and the merge kernel combines the pieces of an
// item exactly in powers of two.  The repair tiles need every item's final
// maximum, so workspaces with a repair set are not split.
//
// A short launch -- at most kAttnSlots query blocks in all, of two 16-tile
// groups per item (2048 < S <= 4096) -- runs `halves` instead: one workgroup
// per query block, its waves in two halves over key tiles [0, 16) and
// [16, nblk), merged inside the workgroup; no partial slots and no merge
// launch.  (Each half streams its own K and V tiles, twice the tile copies
// per step of the cut form, which costs more than the merge saves once the
// halves are longer than one group.)
constexpr int kAttnSlots = 256;           // MI355X compute units
constexpr int kAttnGroup = 16;            // tiles per piece-boundary group
struct AttnSplit {
  int64_t items;      // work items
  int64_t whole;      // items run whole (a multiple of kAttnSlots, or all)
  int tail;           // items cut into pieces
  int tail_wg;        // workgroups over the cut items
  int per;            // groups per tail workgroup
  int ngrp;           // groups per item
  int halves;         // 1: the short-launch form, B*H*nblk workgroups
  int ka;             // its first half's tiles
};
__host__ __device__ inline AttnSplit attn_split(int64_t BH, int nblk, int nrep) {
  AttnSplit p;
  p.items = BH * ((nblk + 1) / 2);
  p.ngrp = (nblk + kAttnGroup - 1) / kAttnGroup;
  p.whole = p.items;
  p.tail = p.tail_wg = p.per = p.halves = p.ka = 0;
  const int R = static_cast<int>(p.items % kAttnSlots);
  if (nrep > 0 || R == 0 || p.ngrp < 2) return p;
  const int per = static_cast<int>((static_cast<int64_t>(R) * p.ngrp + kAttnSlots - 1) / kAttnSlots);
  if (p.ngrp == 2 && BH * nblk <= kAttnSlots) {
    p.whole = 0;
    p.halves = 1;
    p.ka = kAttnGroup;
    return p;
  }
  if (per >= p.ngrp) return p;           // no group saved per compute unit
  p.whole = p.items - R;
  p.tail = R;
  p.per = per;
  p.tail_wg = static_cast<int>((static_cast<int64_t>(R) * p.ngrp + per - 1) / per);
  return p;
}
// A partial slot: O [256 queries][128 channels], then the row sums l [256]
// and the reference exponents [256] (the integer running maximum M, or the
// MXFP4 anchor A), all fp32; two slots per tail workgroup.
constexpr int kPartFloats = 256 * kD + 2 * 256;
constexpr size_t kPartBytes = sizeof(float) * kPartFloats;

// k-means per-cluster sums of the sketch (|x| <= 255) reach 255 * S in
// magnitude: 32-bit while S <= 2^23 (255 * 2^23 < 2^31), 64-bit beyond.  The
// scratch holds the 64-bit width; the 32-bit sums use its first half.
__host__ __device__ inline bool wide_sums(int S) { return S > (1 << 23); }

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

// ---- input loads ------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(b)));
}

// Load 8 consecutive elements (16 bytes, 16-byte aligned) as float.
__device__ __forceinline__ void load8(const void* base, int64_t off, int dtype, float* out) {
  const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  if (dtype == VC_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      out[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = f16_bits_to_f32(w[i] & 0xFFFFu);
      out[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
    }
  }
}

// load8 for an input type fixed at compile time (no branch on the type)
template <int DT>
__device__ __forceinline__ void load8_t(const void* base, int64_t off, float* out) {
  const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (DT == VC_BF16) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    } else {
      out[2 * i] = f16_bits_to_f32(w[i] & 0xFFFFu);
      out[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
    }
  }
}

__device__ __forceinline__ float load1(const void* base, int64_t off, int dtype) {
  const uint32_t b = reinterpret_cast<const uint16_t*>(base)[off];
  return dtype == VC_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Four finite values -> four OCP E4M3 codes, packed little-endian, with
// gfx950's conversion instruction (round half to even).  For finite inputs
// of magnitude <= 448 it gives the same bytes as e4m3_encode below -- checked
// on the device over 2^31 inputs that include every midpoint between
// neighbouring codes, denormals and signed zeros; the quantisers only feed it
// x * (448 / amax) with |x| <= amax.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// ---- OCP E4M3FN encode: round half to even, saturate to +-448 ----------------
// The sign bit follows the input's sign, also when the magnitude rounds to 0.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {                       // below 2^-6: quantum 2^-9 (subnormal codes)
    return sign | static_cast<uint32_t>(rintf(a * 512.0f));
  }
  const int e = static_cast<int>(__float_as_uint(a) >> 23) - 127;   // floor(log2 a), -6..8
  const uint32_t m = static_cast<uint32_t>(rintf(ldexpf(a, 3 - e)));   // 8..16, exact scaling
  const uint32_t code = static_cast<uint32_t>((e + 7) * 8) + (m - 8u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// E4M3 decode (finite codes).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? static_cast<float>(m) * 0.001953125f
                           : ldexpf(1.0f + static_cast<float>(m) * 0.125f, static_cast<int>(e) - 7);
  return (c & 0x80u) ? -mag : mag;
}

// ---- packed tile offsets (see vc.h) -----------------------------------------
// Row tile: operand rows of 16, two 16-byte halves of each 32-byte lane slice.
__device__ __forceinline__ int row_tile_off(int r, int d) {
  return ((((r >> 4) * 2 + ((d & 31) >> 4)) * 64 + (r & 15) + 16 * (d >> 5)) << 4) + (d & 15);
}
// MXFP4 workspaces relabel the keys of every tile so that each FP4 operand
// lane group of the P.V product holds one MXFP4 scale group, a run of 32
// consecutive permuted positions: key slot r = 16t + 4g + i (row r of the K
// tile, key i of lane group g in score sub-tile t) holds permuted position
// 64(t/4) + 16g + 4(t%4) + i of the tile.  Non-causal attention does not
// depend on the order of keys within a tile, so only the storage changes.
__host__ __device__ inline int mx_pos_of_slot(int r) {
  const int t = r >> 4, g = (r >> 2) & 3, i = r & 3;
  return 64 * (t >> 2) + 16 * g + 4 * (t & 3) + i;
}
// Transposed tile: key j and channel d, in the P^T slot order of the score
// accumulator (16x16 MFMA output rows 4g..4g+3 of key sub-tile t).
__device__ __forceinline__ int tr_tile_off(int j, int d) {
  const int g = (j & 15) >> 2;
  const int i = 4 * (j >> 4) + (j & 3);
  return ((((d >> 4) * 2 + (i >> 4)) * 64 + (d & 15) + 16 * g) << 4) + (i & 15);
}

// ---- reductions ---------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap instructions (VALU, no LDS round trip).
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Max over a block of blockDim.x threads (multiple of 64); `red` holds >= 16 floats.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}

// Splitmix64 output for one state value (Vigna's public definition).
__device__ __host__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Workspace scratch (k-means state, sort counters, repair scores), offsets
// relative to the scratch region; computed identically on host and device.
struct Scratch {
  size_t cent, cent_op, cnorm, csum, ccount, chunk_hist, chunk_off, rep_norm, rep_sel, total;
};
// Centroid operands of the assignment MFMA, per (b,h): [4 ct][4 kk][64 lanes]
// x 16 bytes (8 bf16 values: centroid 16ct + lane%16, dims 32kk + 8(lane/16) + i).
constexpr int kCentOpBytes = 4 * 4 * 64 * 16;

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

__host__ __device__ inline Scratch scratch_layout(int64_t BH, int S, int k, int nrep) {
  Scratch s;
  size_t o = 0;
  const int asg = asg_tokens(BH, S);
  const int64_t nchunk = (S + asg - 1) / asg;
  s.cent = o;        o = align256(o + sizeof(int32_t) * BH * k * kD);
  s.cent_op = o;     o = align256(o + static_cast<size_t>(BH) * kCentOpBytes);
  s.cnorm = o;       o = align256(o + sizeof(int32_t) * BH * kMaxK);
  s.csum = o;        o = align256(o + sizeof(int64_t) * BH * k * kD);
  s.ccount = o;      o = align256(o + sizeof(int32_t) * BH * k);
  s.chunk_hist = o;  o = align256(o + sizeof(int32_t) * BH * nchunk * k);
  s.chunk_off = o;   o = align256(o + sizeof(int32_t) * BH * nchunk * k);
  s.rep_norm = o;    o = align256(o + (nrep > 0 ? sizeof(double) * BH * S : 0));
  s.rep_sel = o;     o = align256(o + (nrep > 0 ? sizeof(int32_t) * BH * 4 : 0));
  s.total = o;
  return s;
}

}  // namespace vc

// vc_prepare.hip -- prepare kernels for the VC-Attention forward (gfx950).
//
// V-Smooth ("VC-Attention: Value Smoothing and Softmax Casting for Low-bit
// Attention", Abstract; "Nunchux AI lanza VC-Attention kernel ...",
// paragraph 2): value tokens of each (batch, head) are clustered by k-means
// and reordered by cluster; each 128-position block's mean is subtracted and
// only the residual is quantised to E4M3 with one scale per head ("Open VC
// Attention", Description).  K is gathered through the same permutation so
// keys stay paired with values (non-causal attention is invariant to a joint
// key/value reordering); Q keeps its order.  Q and K get one E4M3 scale per
// 128-token block.
//
// The clustering runs on an integer sketch of V (V scaled by an exact power
// of two and rounded to [-255, 255]); every distance, sum and count is an
// exact integer, so assignments and the permutation do not depend on
// summation order.  All kernels are HBM-bound streaming passes; the k-means
// distances run on the bf16 matrix core (exact for these integers).
#include "vc_common.hpp"
#include "vc_kernels.hpp"

namespace vc {

// ---------------------------------------------------------------------------
__global__ void k_fill_u32(uint32_t* p, uint32_t value, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// max|v| over each (b,h).  grid (ceil(S/kAbsTok), H, B), 256 threads.
// The maximum is taken on the magnitude bits: for finite fp16 and bf16
// values, |x| orders as its 15 low bits do, so one conversion per workgroup
// gives exactly max|v|.
constexpr int kAbsTok = 256;          // tokens per workgroup (16 per pass of 256 threads)
__global__ void __launch_bounds__(256) k_v_absmax(TensorArg v, int S, vc_head_hdr* hdr) {
  __shared__ uint32_t red[4];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y;
  const int s0 = blockIdx.x * kAbsTok;
  const uint16_t* base = reinterpret_cast<const uint16_t*>(v.p) + b * v.sB + h * v.sH + 8 * (threadIdx.x & 15);
  // all loads first (rows past S re-read row S-1 of the same head, which
  // leaves the maximum unchanged), then the maxima
  uint4 raw[kAbsTok / 16];
#pragma unroll
  for (int it = 0; it < kAbsTok / 16; ++it) {
    const int s = min(s0 + it * 16 + static_cast<int>(threadIdx.x >> 4), S - 1);
    raw[it] = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(s) * v.sS);
  }
  uint32_t m = 0;
#pragma unroll
  for (int it = 0; it < kAbsTok / 16; ++it) {
    const uint32_t w[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o, 64)));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const float a = v.dtype == VC_BF16 ? bf16_bits_to_f32(m) : f16_bits_to_f32(m);
    if (a > 0.0f) atomicMax(&hdr[b * H + h].v_amax_bits, __float_as_uint(a));
  }
}

__device__ __forceinline__ float sketch1(float x, int shift) {
  return fminf(fmaxf(rintf(ldexpf(x, shift)), -255.0f), 255.0f);
}

// Centroid operands and squared norms for the assignment pass, from the
// integer centroids of one (b,h) (exact: |c| <= 255 fits bf16, norms < 2^24).
// Called by a whole block after the centroids are final; `nthr` threads.
__device__ void write_cent_ops(int bh, int k, const int32_t* cg, uint8_t* cent_op, int32_t* cnorm, int nthr,
                               int c0 = 0, int c1 = kMaxK) {
  // operands and norms of centroids c0 .. c1-1 (c >= k: absent, zero operand)
  uint8_t* op = cent_op + static_cast<int64_t>(bh) * kCentOpBytes;
  for (int u = threadIdx.x; u < 4 * 4 * 64; u += nthr) {
    const int ct = u >> 8, kk = (u >> 6) & 3, lane = u & 63;
    const int c = 16 * ct + (lane & 15), d0 = 32 * kk + 8 * (lane >> 4);
    if (c < c0 || c >= c1) continue;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = c < k ? static_cast<float>(cg[c * kD + d0 + 2 * i]) : 0.0f;
      const float hi = c < k ? static_cast<float>(cg[c * kD + d0 + 2 * i + 1]) : 0.0f;
      w[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);   // exact: small integers
    }
    *reinterpret_cast<uint4*>(op + static_cast<int64_t>(u) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // squared norms, one wave per centroid at a time: lane l adds dims 2l, 2l+1
  // (exact integers, so the order of the sum does not matter)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nwv = nthr >> 6;
  for (int c = c0 + wv; c < c1; c += nwv) {
    int32_t n2 = 0x7FFFFFFF;                    // absent centroid: never the minimum
    if (c < k) {
      const int32_t a = cg[c * kD + 2 * lane], b = cg[c * kD + 2 * lane + 1];
      n2 = a * a + b * b;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) n2 += __shfl_xor(n2, o, 64);
    }
    if (lane == 0) cnorm[bh * kMaxK + c] = n2;
  }
}

// Sketch shift and seeded strided initial centroids.  grid (BH), 256 threads.
__global__ void __launch_bounds__(256) k_kmeans_init(TensorArg v, int S, int H, int k, uint64_t seed,
                                                     vc_head_hdr* hdr, int32_t* cent, int32_t* csum,
                                                     int32_t* ccount, uint8_t* cent_op, int32_t* cnorm) {
  const int bh = blockIdx.x, b = bh / H, h = bh % H, tid = threadIdx.x;
  const float a = __uint_as_float(hdr[bh].v_amax_bits);
  int shift = 0;
  if (a > 0.0f) {
    int e;
    frexpf(a, &e);              // a in [2^(e-1), 2^e)
    shift = 8 - e;              // 7 - floor(log2 a)
  }
  if (tid == 0) hdr[bh].shift = shift;
  const int stride = S / k > 1 ? S / k : 1;
  const int phi = static_cast<int>(splitmix64(seed ^ static_cast<uint64_t>(bh)) % static_cast<uint64_t>(stride));
  // (centroid c, dim d) pairs i = 128c + d, 32 per thread; every load is
  // issued before the first store (c*S < 2^31 for S <= 2^24, k <= 64)
  constexpr int kPer = kMaxK * kD / 256;
  float xs[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + 256 * j, c = i >> 7, d = i & (kD - 1);
    const int t = (c * S) / k + phi;
    xs[j] = c < k ? load1(v.p, b * v.sB + static_cast<int64_t>(t) * v.sS + h * v.sH + d, v.dtype) : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + 256 * j, c = i >> 7;
    if (c < k) {
      cent[static_cast<int64_t>(bh) * k * kD + i] = static_cast<int32_t>(sketch1(xs[j], shift));
      csum[static_cast<int64_t>(bh) * k * kD + i] = 0;
    }
  }
  if (tid < k) ccount[bh * k + tid] = 0;
  __syncthreads();
  write_cent_ops(bh, k, cent + static_cast<int64_t>(bh) * k * kD, cent_op, cnorm, 256);
}

// One Lloyd assignment pass over asg (asg_tokens: 256..1024) tokens per workgroup.
//   ACCUM: add the block's per-cluster sketch sums and counts to csum/ccount.
//   FINAL: write assign[] and the block's cluster histogram (for the sort).
// Distances run on the matrix core: scores^T = C . X^T with
// v_mfma_f32_16x16x32_bf16, centroids as the A operand (held in registers
// for the whole block), 16 tokens as the B operand.  Sketch values and
// centroids are integers in [-255, 255], exact in bf16; every dot product
// is an integer below 2^24, so the fp32 accumulation is exact in any order.
// Lane l then holds the scores of centroids 16ct + 4(l/16) + i for token
// l%16: an in-lane argmin over its centroids and a 4-lane combine give the
// cluster, ties to the lowest index.  grid (ceil(S/asg), H, B), 256 threads.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
constexpr int kSumPitch = kD + 1;   // padded LDS pitch of the per-cluster sums

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw 16-byte loads of one token-tile iteration (16 tokens per wave, lane
// group g holds dims 32kk + 8g..8g+7).
struct TokRaw {
  uint4 r[4];
};
__device__ __forceinline__ TokRaw load_tok(const TensorArg& v, int b, int h, int tok, bool valid, int g) {
  TokRaw t;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    t.r[kk] = valid ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(v.p) + b * v.sB +
                                                      static_cast<int64_t>(tok) * v.sS + h * v.sH + 32 * kk + 8 * g)
                    : make_uint4(0, 0, 0, 0);
  return t;
}
// fp16/bf16 element -> sketch value (an integer in [-255, 255]) as bf16 bits
__device__ __forceinline__ uint32_t sketch_bits(uint32_t e16, int dtype, int shift) {
  const float x = dtype == VC_BF16 ? __uint_as_float(e16 << 16) : f16_bits_to_f32(e16);
  const float s = __builtin_amdgcn_fmed3f(rintf(ldexpf(x, shift)), -255.0f, 255.0f);
  return __float_as_uint(s) >> 16;           // exact: at most 8 significant bits
}

template <bool ACCUM, bool FINAL, int NCT>
__global__ void __launch_bounds__(256) k_kmeans_assign(TensorArg v, int S, int k, int asg, const vc_head_hdr* hdr,
                                                       const uint8_t* cent_op, const int32_t* cnorm,
                                                       int32_t* csum, int32_t* ccount, int32_t* assign,
                                                       int32_t* chunk_hist) {
  __shared__ int32_t sums[ACCUM ? kMaxK * kSumPitch : 1];
  __shared__ int32_t cnt[kMaxK];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int shift = hdr[bh].shift;
  if (ACCUM)
    for (int i = tid; i < k * kSumPitch; i += 256) sums[i] = 0;
  if (tid < kMaxK) cnt[tid] = 0;
  // centroid operands (prepared with the centroids) and norms
  v8bf ca[NCT][4];
  const uint8_t* op = cent_op + static_cast<int64_t>(bh) * kCentOpBytes;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      ca[ct][kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(op + ((ct * 4 + kk) * 64 + lane) * 16));
  int32_t cn[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) cn[ct][i] = cnorm[bh * kMaxK + 16 * ct + 4 * g + i];
  __syncthreads();

  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const int s0 = blockIdx.x * asg;
  const int kIters = asg / 64;
  int tok = s0 + w * 16 + l16;
  TokRaw nxt = load_tok(v, b, h, tok, tok < S, g);
  for (int tt = 0; tt < kIters; ++tt) {
    const TokRaw cur = nxt;
    const bool valid = tok < S;
    const int tok_next = tok + 64;
    if (tt + 1 < kIters) nxt = load_tok(v, b, h, tok_next, tok_next < S, g);   // one iteration ahead
    v8bf xb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t wv[4] = {cur.r[kk].x, cur.r[kk].y, cur.r[kk].z, cur.r[kk].w};
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk[i] = sketch_bits(wv[i] & 0xFFFFu, v.dtype, shift) | (sketch_bits(wv[i] >> 16, v.dtype, shift) << 16);
      xb[kk] = __builtin_bit_cast(v8bf, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
    v4f acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = zero;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] = mfma_bf16(ca[ct][kk], xb[kk], acc[ct]);
    int32_t best = 0x7FFFFFFF;
    int bc = 0;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cn[ct][i] != 0x7FFFFFFF) {
          const int32_t sc = cn[ct][i] - 2 * static_cast<int32_t>(acc[ct][i]);
          if (sc < best) {
            best = sc;
            bc = 16 * ct + 4 * g + i;
          }
        }
      }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const int32_t ob = __shfl_xor(best, off, 64);
      const int oc = __shfl_xor(bc, off, 64);
      if (ob < best || (ob == best && oc < bc)) {
        best = ob;
        bc = oc;
      }
    }
    if (valid) {
      if (g == 0) {
        atomicAdd(&cnt[bc], 1);
        if (FINAL) assign[static_cast<int64_t>(bh) * S + tok] = bc;
      }
      if (ACCUM) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            atomicAdd(&sums[bc * kSumPitch + 32 * kk + 8 * g + i], static_cast<int32_t>(static_cast<float>(xb[kk][i])));
      }
    }
    tok = tok_next;
  }
  __syncthreads();
  if (ACCUM) {
    int32_t* gs = csum + static_cast<int64_t>(bh) * k * kD;
    for (int i = tid; i < k * kD; i += 256) {
      const int32_t val = sums[(i / kD) * kSumPitch + (i % kD)];
      if (val != 0) atomicAdd(&gs[i], val);
    }
    if (tid < k && cnt[tid] != 0) atomicAdd(&ccount[bh * k + tid], cnt[tid]);
  }
  if (FINAL && tid < k) {
    const int nchunk = (S + asg - 1) / asg;
    chunk_hist[(static_cast<int64_t>(bh) * nchunk + blockIdx.x) * k + tid] = cnt[tid];
  }
}

// New centroid = floor((2*sum + n) / (2n)) (mean rounded half up); empty
// clusters keep their centroid; sums and counts are cleared for the next pass.
// The quotient is taken in fp64: |2*sum + n| < 2^53, so the correctly rounded
// fp64 quotient lies on the same side of every integer as the exact one
// (|q| <= 255 and a non-integer quotient is >= 1/(2n) >= 2^-25 from one).
// grid (BH, ceil(k/8)), 256 threads; a workgroup owns 8 centroids.
constexpr int kUpdCent = 8;
__global__ void __launch_bounds__(256) k_kmeans_update(int k, int32_t* cent, int32_t* csum, int32_t* ccount,
                                                      uint8_t* cent_op, int32_t* cnorm) {
  const int bh = blockIdx.x;
  const int c0 = blockIdx.y * kUpdCent, c1 = c0 + kUpdCent < k ? c0 + kUpdCent : k;
  int32_t* cg = cent + static_cast<int64_t>(bh) * k * kD;
  int32_t* sg = csum + static_cast<int64_t>(bh) * k * kD;
  for (int i = c0 * kD + threadIdx.x; i < c1 * kD; i += blockDim.x) {
    const int32_t n = ccount[bh * k + i / kD];
    if (n > 0) {
      const int64_t num = 2 * static_cast<int64_t>(sg[i]) + n;
      cg[i] = static_cast<int32_t>(floor(static_cast<double>(num) / static_cast<double>(2 * n)));
    }
    sg[i] = 0;
  }
  __syncthreads();
  if (threadIdx.x < c1 - c0) ccount[bh * k + c0 + threadIdx.x] = 0;
  write_cent_ops(bh, k, cg, cent_op, cnorm, 256, c0, c1);
}

// Per-cluster start offsets and per-chunk offsets for the stable scatter.
// grid (BH), 64 * kScanRows threads: thread (r, c) = (tid / 64, tid % 64)
// walks row r, one contiguous range of chunks, for cluster c -- once to total
// it, once to write the offsets; integer sums, so any split gives the same
// offsets as one walk over all chunks.
constexpr int kScanRows = 16;
__global__ void __launch_bounds__(64 * kScanRows) k_cluster_scan(int S, int k, int asg, const int32_t* chunk_hist,
                                                                 int32_t* chunk_off) {
  __shared__ int32_t part[kScanRows][kMaxK];
  __shared__ int32_t tot[kMaxK];
  const int bh = blockIdx.x, c = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int nchunk = (S + asg - 1) / asg;
  const int per = (nchunk + kScanRows - 1) / kScanRows;
  const int j0 = min(r * per, nchunk), j1 = min(j0 + per, nchunk);
  const int32_t* hst = chunk_hist + static_cast<int64_t>(bh) * nchunk * k;
  int32_t* off = chunk_off + static_cast<int64_t>(bh) * nchunk * k;
  int32_t t = 0;
  if (c < k)
    for (int j = j0; j < j1; ++j) t += hst[j * k + c];
  part[r][c] = t;
  __syncthreads();
  if (r == 0) {
    int32_t sum = 0;
    for (int i = 0; i < kScanRows; ++i) sum += part[i][c];
    tot[c] = sum;
  }
  __syncthreads();
  if (c < k) {
    int32_t run = 0;
    for (int j = 0; j < c; ++j) run += tot[j];          // clusters before c
    for (int i = 0; i < r; ++i) run += part[i][c];      // earlier rows of cluster c
    for (int j = j0; j < j1; ++j) {
      off[j * k + c] = run;
      run += hst[j * k + c];
    }
  }
}

// Stable counting-sort scatter: perm[pos] = token, ordered by (cluster, token).
// One asg-token chunk per workgroup, walked in token order in passes of
// 256; ranks within a wave come from ballots.  grid (ceil(S/1024), H, B),
// 256 threads.
__global__ void __launch_bounds__(256) k_cluster_scatter(int S, int k, int asg, const int32_t* assign,
                                                         const int32_t* chunk_off, int32_t* perm) {
  __shared__ int32_t wcount[4][kMaxK];
  __shared__ int32_t run[kMaxK];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nchunk = (S + asg - 1) / asg;
  const int32_t* off = chunk_off + (static_cast<int64_t>(bh) * nchunk + blockIdx.x) * k;
  if (tid < kMaxK) run[tid] = 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int it = 0; it < asg / 256; ++it) {
    for (int i = tid; i < 4 * kMaxK; i += 256) (&wcount[0][0])[i] = 0;
    __syncthreads();
    const int s = blockIdx.x * asg + it * 256 + tid;
    const bool valid = s < S;
    const int c = valid ? assign[static_cast<int64_t>(bh) * S + s] : -1;
    uint64_t rem = __ballot(valid);
    int rank = 0;
    while (rem) {
      const int leader = __ffsll(static_cast<unsigned long long>(rem)) - 1;
      const int cl = __builtin_amdgcn_readlane(c, leader);
      const uint64_t m = __ballot(valid && c == cl);
      if (valid && c == cl) rank = __popcll(m & lt);
      if (lane == 0) wcount[w][cl] = __popcll(m);
      rem &= ~m;
    }
    __syncthreads();
    if (valid) {
      int pos = off[c] + run[c] + rank;
      for (int j = 0; j < w; ++j) pos += wcount[j][c];
      perm[static_cast<int64_t>(bh) * S + pos] = s;
    }
    __syncthreads();
    if (tid < k) run[tid] += wcount[0][tid] + wcount[1][tid] + wcount[2][tid] + wcount[3][tid];
    __syncthreads();
  }
}

// smooth = 0: identity order, cluster 0.  grid (ceil(S/256), H, B).
__global__ void k_identity_perm(int S, int32_t* assign, int32_t* perm) {
  const int bh = blockIdx.z * gridDim.y + blockIdx.y;
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S) {
    perm[static_cast<int64_t>(bh) * S + s] = s;
    assign[static_cast<int64_t>(bh) * S + s] = 0;
  }
}

// Block means over permuted positions and the residual amax per head.
// mu = fp32(fp64(sum) / n), the sum in position order; R = fp32(v - mu).
// The block's gathered rows are read once, 16 bytes per load, into LDS.
// grid (nblk, H, B), 256 threads.
__global__ void __launch_bounds__(256) k_v_block_stats(TensorArg v, int S, int smooth, const int32_t* perm,
                                                       float* v_mean, vc_head_hdr* hdr) {
  __shared__ uint4 rows[kBlock][kD / 8];      // raw 16-bit values of the block's rows
  __shared__ int32_t pp[kBlock];
  __shared__ float red[16];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h, blk = blockIdx.x;
  const int tid = threadIdx.x;
  const int p0 = blk * kBlock;
  const int n = S - p0 < kBlock ? S - p0 : kBlock;
  if (tid < n) pp[tid] = perm[static_cast<int64_t>(bh) * S + p0 + tid];
  __syncthreads();
  for (int t = tid; t < n * (kD / 8); t += blockDim.x) {
    const int j = t >> 4, c8 = (t & 15) * 8;
    rows[j][t & 15] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(v.p) + b * v.sB +
                                                      static_cast<int64_t>(pp[j]) * v.sS + h * v.sH + c8);
  }
  __syncthreads();
  float m = 0.0f;
  if (tid < kD) {
    const int d = tid;
    const uint16_t* col = reinterpret_cast<const uint16_t*>(&rows[0][0]) + d;
    float mu = 0.0f;
    if (smooth) {
      double sum = 0.0;
      for (int j = 0; j < n; ++j) {
        const uint32_t e = col[j * kD];
        sum += static_cast<double>(v.dtype == VC_BF16 ? bf16_bits_to_f32(e) : f16_bits_to_f32(e));
      }
      mu = static_cast<float>(sum / static_cast<double>(n));
    }
    v_mean[(static_cast<int64_t>(bh) * gridDim.x + blk) * kD + d] = mu;
    for (int j = 0; j < n; ++j) {
      const uint32_t e = col[j * kD];
      const float x = v.dtype == VC_BF16 ? bf16_bits_to_f32(e) : f16_bits_to_f32(e);
      m = fmaxf(m, fabsf(x - mu));
    }
  }
  m = block_max(m, red);
  if (tid == 0 && m > 0.0f) atomicMax(&hdr[bh].r_amax_bits, __float_as_uint(m));
}

__device__ __forceinline__ void v_scales(const vc_head_hdr& hd, float* s, float* inv) {
  const float a = __uint_as_float(hd.r_amax_bits);
  *inv = a > 0.0f ? 448.0f / a : 1.0f;
  *s = a > 0.0f ? a / 448.0f : 1.0f;
}

// Gather a 128x128 code block into a transposed (P^T slot order) tile.
__device__ __forceinline__ void store_tr_tile(const uint8_t* codes /*[128][128] in LDS*/, uint8_t* dst) {
  for (int ch = threadIdx.x; ch < kTileBytes / 16; ch += blockDim.x) {
    const int lane = ch & 63, hh = (ch >> 6) & 1, dt = ch >> 7;
    const int g = lane >> 4, d = 16 * dt + (lane & 15);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bi = 16 * hh + 4 * q + e;                    // slot byte 0..31
        const int j = 16 * (bi >> 2) + 4 * g + (bi & 3);       // key within the tile
        word |= static_cast<uint32_t>(codes[j * kD + d]) << (8 * e);
      }
      w[q] = word;
    }
    *reinterpret_cast<uint4*>(dst + ch * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// E4M3 residual codes, written as transposed tiles; mu' = mu / s_v.
// grid (nblk, H, B), 256 threads.
__global__ void __launch_bounds__(256) k_v_quant_pack(TensorArg v, int S, const int32_t* perm, const float* v_mean,
                                                      vc_head_hdr* hdr, uint8_t* v8, uint8_t* v_muop) {
  __shared__ __align__(16) uint8_t codes[kTileBytes];
  __shared__ float mu[kD];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h, blk = blockIdx.x, nblk = gridDim.x;
  float s_v, inv;
  v_scales(hdr[bh], &s_v, &inv);
  if (threadIdx.x < kD) {
    const int ch = threadIdx.x;
    const float m = v_mean[(static_cast<int64_t>(bh) * nblk + blk) * kD + ch];
    mu[ch] = m;
    // restore operand: mu/s_v split into bf16 high and low parts
    const float mp = m / s_v;
    const uint16_t hi = static_cast<uint16_t>(f32_to_bf16_bits(mp));
    const uint16_t lo = static_cast<uint16_t>(f32_to_bf16_bits(mp - __uint_as_float(static_cast<uint32_t>(hi) << 16)));
    const int p = blk % kMuOpGroup, row = (blk - p) + 2 * (ch >> 4);
    const int off = ((p >> 2) * 16 + (ch & 15)) * 8 + (p & 3) * 2;
    uint8_t* base = v_muop + static_cast<int64_t>(bh) * muop_rows(nblk) * kMuOpRowBytes;
    *reinterpret_cast<uint16_t*>(base + static_cast<int64_t>(row) * kMuOpRowBytes + off) = hi;
    *reinterpret_cast<uint16_t*>(base + static_cast<int64_t>(row + 1) * kMuOpRowBytes + off) = lo;
  }
  if (blk == 0 && threadIdx.x == 0) {
    hdr[bh].v_scale = s_v;
    hdr[bh].v_inv = inv;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < kBlock * 16; t += blockDim.x) {
    const int j = t >> 4, c8 = (t & 15) * 8;
    const int p = blk * kBlock + j;
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (p < S) {
      const int s = perm[static_cast<int64_t>(bh) * S + p];
      float x[8], r[8];
      load8(v.p, b * v.sB + s * v.sS + h * v.sH + c8, v.dtype, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (x[e] - mu[c8 + e]) * inv;
      c[0] = e4m3_pack4(r[0], r[1], r[2], r[3]);
      c[1] = e4m3_pack4(r[4], r[5], r[6], r[7]);
    }
    *reinterpret_cast<uint2*>(&codes[j * kD + c8]) = make_uint2(c[0], c[1]);
  }
  __syncthreads();
  store_tr_tile(codes, v8 + (static_cast<int64_t>(bh) * nblk + blk) * kTileBytes);
}

// MXFP4 residual ("Nunchux AI lanza VC-Attention kernel ...", paragraph 2:
// a 4-bit residual beside E4M3; taken as OCP MXFP4 for the gfx950 matrix
// core): R = fp32(v - mu), one E8M0 scale per channel and group of 32 keys
// -- the keys one matrix-core lane holds as an FP4 operand -- chosen as the
// smallest power of two X with max|R|/X <= 6, and E2M1 codes of R/X (round
// half to even, sign from R).  No per-head scale (s_v = 1, mu' = mu).
// grid (nblk, H, B), 256 threads; thread = 2 (channel, group) pairs.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
  const float a = fabsf(y);
  // thresholds of round half to even on the grid 0, .5, 1, 1.5, 2, 3, 4, 6
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
                     (a > 5.0f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}
// Smallest e with amax <= 6 * 2^e, for amax = m * 2^k (m in [0.5, 1)):
// e = k - 3 when m <= 0.75, else k - 2; 0 for amax == 0; clamped to the
// E8M0 range.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int k;
  const float m = frexpf(amax, &k);
  const int e = k - (m <= 0.75f ? 3 : 2);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
__global__ void __launch_bounds__(256) k_v_quant_pack_fp4(TensorArg v, int S, const int32_t* perm,
                                                          const float* v_mean, vc_head_hdr* hdr, uint8_t* v8,
                                                          uint8_t* v_muop) {
  __shared__ float res[kBlock][kD + 1];   // residual of the tile (padded rows against bank conflicts)
  __shared__ float mu[kD];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h, blk = blockIdx.x, nblk = gridDim.x;
  if (threadIdx.x < kD) {
    const int ch = threadIdx.x;
    const float m = v_mean[(static_cast<int64_t>(bh) * nblk + blk) * kD + ch];
    mu[ch] = m;
    // restore operand: mu (s_v = 1) split into bf16 high and low parts
    const uint16_t hi = static_cast<uint16_t>(f32_to_bf16_bits(m));
    const uint16_t lo = static_cast<uint16_t>(f32_to_bf16_bits(m - __uint_as_float(static_cast<uint32_t>(hi) << 16)));
    const int p = blk % kMuOpGroup, row = (blk - p) + 2 * (ch >> 4);
    const int off = ((p >> 2) * 16 + (ch & 15)) * 8 + (p & 3) * 2;
    uint8_t* base = v_muop + static_cast<int64_t>(bh) * muop_rows(nblk) * kMuOpRowBytes;
    *reinterpret_cast<uint16_t*>(base + static_cast<int64_t>(row) * kMuOpRowBytes + off) = hi;
    *reinterpret_cast<uint16_t*>(base + static_cast<int64_t>(row + 1) * kMuOpRowBytes + off) = lo;
  }
  if (blk == 0 && threadIdx.x == 0) {
    hdr[bh].v_scale = 1.0f;
    hdr[bh].v_inv = 1.0f;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < kBlock * 16; t += blockDim.x) {
    const int j = t >> 4, c8 = (t & 15) * 8;
    const int p = blk * kBlock + j;
    float r[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (p < S) {
      const int s = perm[static_cast<int64_t>(bh) * S + p];
      float x[8];
      load8(v.p, b * v.sB + s * v.sS + h * v.sH + c8, v.dtype, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = x[e] - mu[c8 + e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) res[j][c8 + e] = r[e];
  }
  __syncthreads();
  uint8_t* tile = v8 + (static_cast<int64_t>(bh) * nblk + blk) * kTileBytes;
  for (int task = threadIdx.x; task < kD * 4; task += blockDim.x) {
    const int d = task & (kD - 1), u = task >> 7;     // channel, lane group
    // nibble n of lane group u holds P-operand K index kb, which is key
    // 16*((kb%32)/4) + 4*(kb/32) + kb%4
    float amax = 0.0f;
#pragma unroll 8
    for (int n = 0; n < 32; ++n) {
      const int kb = 64 * (u & 1) + 16 * (u >> 1) + 32 * (n >> 4) + (n & 15);
      amax = fmaxf(amax, fabsf(res[16 * ((kb & 31) >> 2) + 4 * (kb >> 5) + (kb & 3)][d]));
    }
    const int e = mx_exponent(amax);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll 8
    for (int n = 0; n < 32; ++n) {
      const int kb = 64 * (u & 1) + 16 * (u >> 1) + 32 * (n >> 4) + (n & 15);
      const float y = ldexpf(res[16 * ((kb & 31) >> 2) + 4 * (kb >> 5) + (kb & 3)][d], -e);
      w[n >> 3] |= e2m1_encode(y) << (4 * (n & 7));
    }
    const int lane = u * 16 + (d & 15), dt = d >> 4;
    *reinterpret_cast<uint4*>(tile + (dt * 64 + lane) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    tile[8192 + lane * 8 + dt] = static_cast<uint8_t>(e + 127);
  }
}

// Per-block amax E4M3 quantisation of 128 rows into a row tile.  GATHER: row
// p is token perm[p] (K); otherwise row p is token p (Q).
// grid (nblk, H, B), 256 threads; 4 (row, 16-channel) tasks per thread.
template <bool GATHER>
__global__ void __launch_bounds__(256) k_quant_rows(TensorArg x, int S, const int32_t* perm, uint8_t* out8,
                                                    float* scale) {
  __shared__ float red[16];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h, blk = blockIdx.x, nblk = gridDim.x;
  float val[4][16];
  float m = 0.0f;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int task = threadIdx.x + 256 * it;
    const int r = task >> 3, c16 = (task & 7) * 16;
    const int p = blk * kBlock + r;
    if (p < S) {
      const int s = GATHER ? perm[static_cast<int64_t>(bh) * S + p] : p;
      const int64_t off = b * x.sB + s * x.sS + h * x.sH + c16;
      load8(x.p, off, x.dtype, &val[it][0]);
      load8(x.p, off + 8, x.dtype, &val[it][8]);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) val[it][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(val[it][e]));
  }
  m = block_max(m, red);
  const float inv = m > 0.0f ? 448.0f / m : 1.0f;
  const float sc = m > 0.0f ? m / 448.0f : 1.0f;
  uint8_t* tile = out8 + (static_cast<int64_t>(bh) * nblk + blk) * kTileBytes;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int task = threadIdx.x + 256 * it;
    const int r = task >> 3, c16 = (task & 7) * 16;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = e4m3_pack4(val[it][4 * q] * inv, val[it][4 * q + 1] * inv, val[it][4 * q + 2] * inv,
                        val[it][4 * q + 3] * inv);
    }
    *reinterpret_cast<uint4*>(tile + row_tile_off(r, c16)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (threadIdx.x == 0) {
    scale[static_cast<int64_t>(bh) * nblk + blk] = sc;
  }
}

// ---------------------------------------------------------------------------
// Residual repair ("Open VC Attention", Description): the quantisation error
// e = fp32(R - fp32(s_v * dec(code))) of the worst-rounded value tokens.
// The codes come from the conversion instruction, exactly as the residual
// quantiser makes them (|r * inv| <= 448 up to one rounding, where it gives
// e4m3_encode's bytes), and go back to fp32 with the widening conversion,
// which is exact.
__device__ __forceinline__ void resid_err(const float* xv /*8*/, const float* mu /*8*/, float s_v, float inv,
                                          float* e /*8*/) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = xv[i] - mu[i];
  const int c0 = static_cast<int>(e4m3_pack4(r[0] * inv, r[1] * inv, r[2] * inv, r[3] * inv));
  const int c1 = static_cast<int>(e4m3_pack4(r[4] * inv, r[5] * inv, r[6] * inv, r[7] * inv));
  const v2f d[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(c0, false), __builtin_amdgcn_cvt_pk_f32_fp8(c0, true),
                    __builtin_amdgcn_cvt_pk_f32_fp8(c1, false), __builtin_amdgcn_cvt_pk_f32_fp8(c1, true)};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float deq = s_v * d[i >> 1][i & 1];
    e[i] = r[i] - deq;
  }
}

// Squared error norm per permuted position (sequential fp64 sum over d).
// The block's gathered rows are staged in LDS first, 16 lanes per row (whole
// rows per load instruction), at a padded pitch; then thread j sums row j in
// channel order.  grid (nblk, H, B), 128 threads.
constexpr int kNormPitch = kD / 8 + 1;   // 16-byte units per LDS row
__global__ void __launch_bounds__(128) k_repair_norm(TensorArg v, int S, const int32_t* perm, const float* v_mean,
                                                     const vc_head_hdr* hdr, double* norm) {
  __shared__ float mu[kD];
  __shared__ int32_t pp[kBlock];
  __shared__ uint4 rows[kBlock * kNormPitch];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h, blk = blockIdx.x;
  const int tid = threadIdx.x;
  const int p0 = blk * kBlock;
  const int n = S - p0 < kBlock ? S - p0 : kBlock;
  mu[tid] = v_mean[(static_cast<int64_t>(bh) * gridDim.x + blk) * kD + tid];
  if (tid < n) pp[tid] = perm[static_cast<int64_t>(bh) * S + p0 + tid];
  __syncthreads();
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(v.p) + b * v.sB + h * v.sH;
  for (int t = tid; t < n * (kD / 8); t += blockDim.x) {
    const int j = t >> 4, c = t & 15;
    rows[j * kNormPitch + c] = *reinterpret_cast<const uint4*>(vb + static_cast<int64_t>(pp[j]) * v.sS + 8 * c);
  }
  __syncthreads();
  if (tid >= n) return;
  float s_v, inv;
  v_scales(hdr[bh], &s_v, &inv);
  double acc = 0.0;
  for (int c = 0; c < kD / 8; ++c) {
    float x[8], e[8];
    load8(&rows[tid * kNormPitch + c], 0, v.dtype, x);
    resid_err(x, mu + 8 * c, s_v, inv, e);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = acc + static_cast<double>(e[i]) * static_cast<double>(e[i]);
  }
  norm[static_cast<int64_t>(bh) * S + p0 + tid] = acc;
}

// Top-nrep positions by error norm (ties to the smaller position), written in
// ascending position order; radix select on the fp64 bit patterns (the norms
// are >= 0, so their bits order like the values).  grid (BH), 256 threads.
constexpr int kSelUnroll = 8;
constexpr int kSelThreads = 1024;     // one workgroup per head
constexpr int kSelWaves = kSelThreads / 64;
__global__ void __launch_bounds__(kSelThreads) k_repair_select(int S, int nrep, int nrep_pad, const double* norm,
                                                       int32_t* rep_pos, vc_head_hdr* hdr) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t suf[256];
  __shared__ uint64_t sh_prefix;
  __shared__ int32_t sh_remaining, sh_sel, sh_cum;
  __shared__ int32_t wsum[2][kSelWaves];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t* key = reinterpret_cast<const uint64_t*>(norm) + static_cast<int64_t>(bh) * S;
  if (tid == 0) {
    sh_prefix = 0;
    sh_remaining = nrep;
    hdr[bh].nrep = nrep;
  }
  uint64_t mask = 0;
  for (int pos = 7; pos >= 0; --pos) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = sh_prefix;
    for (int p0 = 0; p0 < S; p0 += kSelThreads * kSelUnroll) {
      // kSelUnroll keys per thread per memory round trip (the loop bound is
      // uniform, so every lane reaches the ballots)
      uint64_t uu[kSelUnroll];
#pragma unroll
      for (int i = 0; i < kSelUnroll; ++i) {
        const int p = p0 + tid + kSelThreads * i;
        uu[i] = key[min(p, S - 1)];
      }
#pragma unroll
      for (int i = 0; i < kSelUnroll; ++i) {
        const uint64_t u = uu[i];
        const bool act = p0 + tid + kSelThreads * i < S && (u & mask) == prefix;
        const uint32_t bin = static_cast<uint32_t>(u >> (8 * pos)) & 255u;
        // the first active lane's bin takes one add for every lane that
        // shares it (most keys share a few bins in the leading bytes); the
        // rest add 1
        const uint64_t am = __ballot(act);
        if (am) {
          const int leader = __ffsll(static_cast<unsigned long long>(am)) - 1;
          const uint32_t lb = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
          const uint64_t same = __ballot(act && bin == lb);
          if (lane == leader) atomicAdd(&hist[lb], static_cast<uint32_t>(__popcll(same)));
          else if (act && bin != lb) atomicAdd(&hist[bin], 1u);
        }
      }
    }
    __syncthreads();
    // suffix[t] = keys in bins t..255; the selected bin is the highest t with
    // suffix[t] >= remaining (bins above it are all taken)
    if (tid < 256) suf[tid] = hist[tid];
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const uint32_t add = tid + d < 256 ? suf[tid + d] : 0u;
      __syncthreads();
      if (tid < 256) suf[tid] += add;
      __syncthreads();
    }
    if (tid < 256) {
      const int32_t rem = sh_remaining;
      const uint32_t above = tid < 255 ? suf[tid + 1] : 0u;
      if (static_cast<int32_t>(suf[tid]) >= rem && static_cast<int32_t>(above) < rem) {
        sh_sel = tid;
        sh_cum = static_cast<int32_t>(above);
      }
    }
    __syncthreads();
    if (tid == 0) {
      sh_remaining -= sh_cum;
      sh_prefix = prefix | (static_cast<uint64_t>(sh_sel) << (8 * pos));
    }
    mask |= 0xFFull << (8 * pos);
    __syncthreads();
  }
  const uint64_t T = sh_prefix;
  const int32_t need_eq = sh_remaining;   // keys equal to T to take, lowest positions first
  int32_t carry_eq = 0, carry_out = 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* out = rep_pos + static_cast<int64_t>(bh) * nrep_pad;
  uint64_t uu[kSelUnroll];
  for (int base = 0; base < S; base += kSelThreads) {
    const int it = (base / kSelThreads) % kSelUnroll;
    if (it == 0) {
#pragma unroll
      for (int i = 0; i < kSelUnroll; ++i) uu[i] = key[min(base + tid + kSelThreads * i, S - 1)];
    }
    const int p = base + tid;
    uint64_t u = uu[0];
#pragma unroll
    for (int i = 1; i < kSelUnroll; ++i) u = it == i ? uu[i] : u;
    const bool eq = p < S && u == T;
    const uint64_t meq = __ballot(eq);
    if (lane == 0) wsum[0][w] = __popcll(meq);
    __syncthreads();
    int32_t eq_rank = carry_eq + __popcll(meq & lt);
    for (int j = 0; j < w; ++j) eq_rank += wsum[0][j];
    const bool take = p < S && (u > T || (eq && eq_rank < need_eq));
    const uint64_t mt = __ballot(take);
    if (lane == 0) wsum[1][w] = __popcll(mt);
    __syncthreads();
    int32_t idx = carry_out + __popcll(mt & lt);
    for (int j = 0; j < w; ++j) idx += wsum[1][j];
    if (take) out[idx] = p;
    for (int j = 0; j < kSelWaves; ++j) {
      carry_eq += wsum[0][j];
      carry_out += wsum[1][j];
    }
    __syncthreads();
  }
  for (int i = nrep + tid; i < nrep_pad; i += kSelThreads) out[i] = -1;
}

// Largest |e| over the repaired rows.  grid (nrep_pad/128, H, B), 128 threads.
__global__ void __launch_bounds__(128) k_repair_eamax(TensorArg v, int S, int nrep_pad, const int32_t* perm,
                                                      const float* v_mean, const int32_t* rep_pos, vc_head_hdr* hdr) {
  __shared__ float red[16];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h;
  const int nblk = (S + kBlock - 1) / kBlock;
  const int i = blockIdx.x * kBlock + threadIdx.x;
  const int p = rep_pos[static_cast<int64_t>(bh) * nrep_pad + i];
  float m = 0.0f;
  if (p >= 0) {
    const int s = perm[static_cast<int64_t>(bh) * S + p];
    const float* mu = v_mean + (static_cast<int64_t>(bh) * nblk + p / kBlock) * kD;
    float s_v, inv;
    v_scales(hdr[bh], &s_v, &inv);
    for (int c8 = 0; c8 < kD; c8 += 8) {
      float x[8], e[8];
      load8(v.p, b * v.sB + s * v.sS + h * v.sH + c8, v.dtype, x);
      resid_err(x, mu + c8, s_v, inv, e);
#pragma unroll
      for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(e[q]));
    }
  }
  m = block_max(m, red);
  if (threadIdx.x == 0 && m > 0.0f) atomicMax(&hdr[bh].e_amax_bits, __float_as_uint(m));
}

// E4M3 repair residuals as transposed tiles (key = repair index).
// grid (nrep_pad/128, H, B), 256 threads.
__global__ void __launch_bounds__(256) k_repair_epack(TensorArg v, int S, int nrep_pad, const int32_t* perm,
                                                      const float* v_mean, const int32_t* rep_pos, vc_head_hdr* hdr,
                                                      uint8_t* rep_e8) {
  __shared__ __align__(16) uint8_t codes[kTileBytes];
  const int b = blockIdx.z, h = blockIdx.y, H = gridDim.y, bh = b * H + h;
  const int nblk = (S + kBlock - 1) / kBlock;
  const float a = __uint_as_float(hdr[bh].e_amax_bits);
  const float inv_e = a > 0.0f ? 448.0f / a : 1.0f;
  const float s_e = a > 0.0f ? a / 448.0f : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) hdr[bh].rep_scale = s_e;
  float s_v, inv;
  v_scales(hdr[bh], &s_v, &inv);
  for (int t = threadIdx.x; t < kBlock * 16; t += blockDim.x) {
    const int j = t >> 4, c8 = (t & 15) * 8;
    const int p = rep_pos[static_cast<int64_t>(bh) * nrep_pad + blockIdx.x * kBlock + j];
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (p >= 0) {
      const int s = perm[static_cast<int64_t>(bh) * S + p];
      const float* mu = v_mean + (static_cast<int64_t>(bh) * nblk + p / kBlock) * kD;
      float x[8], e[8];
      load8(v.p, b * v.sB + s * v.sS + h * v.sH + c8, v.dtype, x);
      resid_err(x, mu + c8, s_v, inv, e);
#pragma unroll
      for (int q = 0; q < 8; ++q) c[q] = e4m3_encode(e[q] * inv_e);
    }
    *reinterpret_cast<uint2*>(&codes[j * kD + c8]) =
        make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24, c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
  }
  __syncthreads();
  store_tr_tile(codes, rep_e8 + (static_cast<int64_t>(bh) * (nrep_pad / kBlock) + blockIdx.x) * kTileBytes);
}

// Copy the K code rows of the repaired positions into row tiles, with their
// block scales.  grid (nrep_pad/128, H, B), 256 threads.
__global__ void __launch_bounds__(256) k_repair_kpack(int S, int nrep_pad, const int32_t* rep_pos, const uint8_t* k8,
                                                      const float* k_scale, uint8_t* rep_k8, float* rep_ks) {
  const int bh = blockIdx.z * gridDim.y + blockIdx.y;
  const int nblk = (S + kBlock - 1) / kBlock;
  uint8_t* dst = rep_k8 + (static_cast<int64_t>(bh) * (nrep_pad / kBlock) + blockIdx.x) * kTileBytes;
  for (int t = threadIdx.x; t < kBlock * 8; t += blockDim.x) {
    const int r = t >> 3, c16 = (t & 7) * 16;
    const int i = blockIdx.x * kBlock + r;
    const int p = rep_pos[static_cast<int64_t>(bh) * nrep_pad + i];
    uint4 val = make_uint4(0, 0, 0, 0);
    if (p >= 0) {
      const uint8_t* src = k8 + (static_cast<int64_t>(bh) * nblk + p / kBlock) * kTileBytes;
      val = *reinterpret_cast<const uint4*>(src + row_tile_off(p % kBlock, c16));
    }
    *reinterpret_cast<uint4*>(dst + row_tile_off(r, c16)) = val;
    if (c16 == 0) rep_ks[static_cast<int64_t>(bh) * nrep_pad + i] = p >= 0 ? k_scale[static_cast<int64_t>(bh) * nblk + p / kBlock] : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// Host-side launch sequences (called from the C ABI after validation).
#define VC_LAUNCH_CHECK()                                   \
  do {                                                      \
    hipError_t _e = hipGetLastError();                      \
    if (_e != hipSuccess) return _e;                        \
  } while (0)

template <bool ACCUM, bool FINAL>
void launch_assign(dim3 grid, hipStream_t st, const TensorArg& v, int S, int k, int asg, const WsPtrs& ws) {
  const int nct = (k + 15) / 16;     // 1..4 (k <= 64)
#define VC_ASSIGN(N)                                                                                    \
  hipLaunchKernelGGL((k_kmeans_assign<ACCUM, FINAL, N>), grid, dim3(256), 0, st, v, S, k, asg, ws.hdr, ws.cent_op, \
                     ws.cnorm, ws.csum, ws.ccount, ws.assign, ws.chunk_hist)
  if (nct == 1) VC_ASSIGN(1);
  else if (nct == 2) VC_ASSIGN(2);
  else if (nct == 3) VC_ASSIGN(3);
  else VC_ASSIGN(4);
#undef VC_ASSIGN
}

hipError_t launch_prepare_v(const TensorArg& v, int B, int S, int H, const vc_v_opts& o, const WsPtrs& ws,
                            hipStream_t st) {
  const int BH = B * H, nblk = (S + kBlock - 1) / kBlock, k = o.k;
  const dim3 gblk(nblk, H, B);
  hipLaunchKernelGGL(k_fill_u32, dim3(64), dim3(256), 0, st, reinterpret_cast<uint32_t*>(ws.hdr), 0u,
                     static_cast<int64_t>(BH) * (sizeof(vc_head_hdr) / 4));
  VC_LAUNCH_CHECK();
  if (o.smooth) {
    const int asg = asg_tokens(BH, S);
    const int nch = (S + asg - 1) / asg;
    hipLaunchKernelGGL(k_v_absmax, dim3((S + kAbsTok - 1) / kAbsTok, H, B), dim3(256), 0, st, v, S, ws.hdr);
    VC_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_kmeans_init, dim3(BH), dim3(256), 0, st, v, S, H, k, o.seed, ws.hdr, ws.cent, ws.csum,
                       ws.ccount, ws.cent_op, ws.cnorm);
    VC_LAUNCH_CHECK();
    for (int it = 0; it < o.iters; ++it) {
      launch_assign<true, false>(dim3(nch, H, B), st, v, S, k, asg, ws);
      VC_LAUNCH_CHECK();
      hipLaunchKernelGGL(k_kmeans_update, dim3(BH, (k + kUpdCent - 1) / kUpdCent), dim3(256), 0, st, k, ws.cent,
                         ws.csum, ws.ccount, ws.cent_op,
                         ws.cnorm);
      VC_LAUNCH_CHECK();
    }
    launch_assign<false, true>(dim3(nch, H, B), st, v, S, k, asg, ws);
    VC_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_cluster_scan, dim3(BH), dim3(64 * kScanRows), 0, st, S, k, asg, ws.chunk_hist,
                       ws.chunk_off);
    VC_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_cluster_scatter, dim3(nch, H, B), dim3(256), 0, st, S, k, asg, ws.assign, ws.chunk_off,
                       ws.perm);
    VC_LAUNCH_CHECK();
  } else {
    hipLaunchKernelGGL(k_identity_perm, dim3((S + 255) / 256, H, B), dim3(256), 0, st, S, ws.assign, ws.perm);
    VC_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_v_block_stats, gblk, dim3(256), 0, st, v, S, o.smooth, ws.perm, ws.v_mean, ws.hdr);
  VC_LAUNCH_CHECK();
  // restore operands: zero first (blocks past the last stay zero)
  hipLaunchKernelGGL(k_fill_u32, dim3(256), dim3(256), 0, st, reinterpret_cast<uint32_t*>(ws.v_muop), 0u,
                     static_cast<int64_t>(BH) * muop_rows(nblk) * (kMuOpRowBytes / 4));
  VC_LAUNCH_CHECK();
  if (o.v_format == VC_V_MXFP4)
    hipLaunchKernelGGL(k_v_quant_pack_fp4, gblk, dim3(256), 0, st, v, S, ws.perm, ws.v_mean, ws.hdr, ws.v8,
                       ws.v_muop);
  else
    hipLaunchKernelGGL(k_v_quant_pack, gblk, dim3(256), 0, st, v, S, ws.perm, ws.v_mean, ws.hdr, ws.v8, ws.v_muop);
  VC_LAUNCH_CHECK();
  if (ws.nrep > 0) {
    const dim3 grep(ws.nrep_pad / kBlock, H, B);
    hipLaunchKernelGGL(k_repair_norm, gblk, dim3(128), 0, st, v, S, ws.perm, ws.v_mean, ws.hdr, ws.rep_norm);
    VC_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_repair_select, dim3(BH), dim3(kSelThreads), 0, st, S, ws.nrep, ws.nrep_pad, ws.rep_norm,
                       ws.rep_pos, ws.hdr);
    VC_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_repair_eamax, grep, dim3(128), 0, st, v, S, ws.nrep_pad, ws.perm, ws.v_mean, ws.rep_pos,
                       ws.hdr);
    VC_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_repair_epack, grep, dim3(256), 0, st, v, S, ws.nrep_pad, ws.perm, ws.v_mean, ws.rep_pos,
                       ws.hdr, ws.rep_e8);
    VC_LAUNCH_CHECK();
  }
  return hipSuccess;
}

hipError_t launch_prepare_qk(const TensorArg& q, const TensorArg& kt, int B, int S, int H, const WsPtrs& ws,
                             hipStream_t st) {
  const int nblk = (S + kBlock - 1) / kBlock;
  const dim3 gblk(nblk, H, B);
  hipLaunchKernelGGL((k_quant_rows<false>), gblk, dim3(256), 0, st, q, S, ws.perm, ws.q8, ws.q_scale);
  VC_LAUNCH_CHECK();
  hipLaunchKernelGGL((k_quant_rows<true>), gblk, dim3(256), 0, st, kt, S, ws.perm, ws.k8, ws.k_scale);
  VC_LAUNCH_CHECK();
  if (ws.nrep > 0) {
    hipLaunchKernelGGL(k_repair_kpack, dim3(ws.nrep_pad / kBlock, H, B), dim3(256), 0, st, S, ws.nrep_pad,
                       ws.rep_pos, ws.k8, ws.k_scale, ws.rep_k8, ws.rep_ks);
    VC_LAUNCH_CHECK();
  }
  return hipSuccess;
}

}  // namespace vc

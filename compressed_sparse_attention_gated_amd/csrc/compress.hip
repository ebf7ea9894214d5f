// Gated per-channel softmax compressor with its write epilogue (RMSNorm, indexer-K
// projection, RoPE).
//
// Pooling follows [Evolution blog] §4.1 (CSA2: softmax over the m in-block positions of
// each channel, weighted sum of the KV rows, then kv_norm) and [DSA-to-CSA notes]
// eq. (11)-(12) (overlapped variant: 2m candidates, block 0's history masked).  The
// epilogue order - norm, indexer-K projection of the un-rotated entry, then position
// encoding - is the one [Evolution blog] §4.1 describes.
//
// Mapping: a row (one compressed entry) is handled by G = c/8 lanes, 8 channels per lane
// (16-byte bf16 or 32-byte fp32 loads, coalesced across the G lanes).  A workgroup of 256
// threads owns 32 consecutive entries; the per-channel softmax runs online over the
// block's m (or 2m) tokens in fp32 with exp2.  HBM-bound: each token row is read once.

#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWG = 32;
constexpr int kMaxSamples = CSA2_MAX_PACKED_SAMPLES;  // packed samples per call (LDS offsets)

template <typename T>
struct Ld;
template <>
struct Ld<float> {
  static __device__ __forceinline__ void load8(const float* p, float* f) {
    float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  static __device__ __forceinline__ void store8(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
  static __device__ __forceinline__ float scalar(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
};
template <>
struct Ld<uint16_t> {
  static __device__ __forceinline__ void load8(const uint16_t* p, float* f) {
    unpack8(*reinterpret_cast<const uint4*>(p), f);
  }
  static __device__ __forceinline__ void store8(uint16_t* p, const float* f) {
    *reinterpret_cast<uint4*>(p) = pack8(f);
  }
  static __device__ __forceinline__ float scalar(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void store1(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// ------------------------------------------------------------------ cache quantisers
// Every rounding decision below compares a value with a threshold times its scale, and
// each such product is exact in fp32 (at most 8 significant bits), so the bytes written
// are the exact round-to-nearest-even of the fp32 entry values: bit-for-bit what any
// exact implementation of the same rule gives for the same inputs.
//
// E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} (codes 0..7): the midpoints between
// neighbours are the thresholds; at a midpoint the even code wins.
__device__ __forceinline__ uint32_t e2m1_code(float x, float scale) {
  const float a = fabsf(x);
  constexpr float kMid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  uint32_t code = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    const float t = kMid[k] * scale;
    code += (a > t) ? 1u : 0u;
    if (k & 1) code += (a == t) ? 1u : 0u;  // tie between codes k and k+1: k+1 is even
  }
  return (x < 0.f && code != 0) ? (code | 8u) : code;
}
// value of a non-negative OCP E4M3FN byte (0x00..0x7e)
__device__ __forceinline__ float e4m3_value(int b) {
  const int e = b >> 3, m = b & 7;
  return e ? __builtin_amdgcn_ldexpf((float)(8 + m), e - 10) : __builtin_amdgcn_ldexpf((float)m, -9);
}
// E4M3 byte nearest to amax / 6 (ties to the even byte, saturating at 448): the largest
// byte whose value times 6 is <= amax, then the midpoint test against its successor
__device__ __forceinline__ int e4m3_scale_byte(float amax) {
  int lo = 0, hi = 0x7e;
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    const int mid = (lo + hi + 1) >> 1;
    const bool le = 6.0f * e4m3_value(mid) <= amax;
    lo = le ? mid : lo;
    hi = le ? hi : mid - 1;
  }
  if (lo >= 0x7e) return 0x7e;
  const float t = 3.0f * (e4m3_value(lo) + e4m3_value(lo + 1));  // 6 x midpoint
  if (amax > t) return lo + 1;
  if (amax < t) return lo;
  return (lo & 1) ? lo + 1 : lo;
}
// MXFP4 shared exponent of a group with max magnitude amax > 0: floor(log2 amax) - 2,
// clamped to [-127, 127] (read off the fp32 exponent; subnormal amax gives -127)
__device__ __forceinline__ int mx_exponent(float amax) {
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return E == 0 ? -127 : max(E - 129, -127);
}
// max over aligned groups of 32 lanes
__device__ __forceinline__ float max32(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  float a, b;
  pair_xor16(v, &a, &b);
  return fmaxf(a, b);
}

// Packed samples: E[s] = number of entries of the samples before s (each sample of len
// tokens gives floor(len / m) entries), E[ns] the total; an exclusive scan over the
// workgroup (each thread a contiguous run of samples), written to LDS.
// sample s's tokens [lo, lo + len) of an n-token stream: its bounds clamped into [0, n] and
// made non-decreasing, so no access leaves the stream whatever the caller's offsets hold
__device__ __forceinline__ void sample_span(const int32_t* __restrict__ cu, int s, int n, int* lo, int* len) {
  const int a = min(max(cu[s], 0), n);
  const int e = min(max(cu[s + 1], a), n);
  *lo = a;
  *len = e - a;
}
__device__ __forceinline__ int sample_entries(const int32_t* __restrict__ cu, int s, int n, int m) {
  int lo, len;
  sample_span(cu, s, n, &lo, &len);
  return len / m;
}
__device__ __forceinline__ void sample_entry_offsets(const int32_t* __restrict__ cu, int ns, int n, int m, int* E,
                                                     int* tmp) {
  const int t = threadIdx.x;
  const int per = (ns + kThreads - 1) / kThreads;
  const int s0 = t * per;
  int local = 0;
  for (int u = 0; u < per; ++u) {
    const int s = s0 + u;
    if (s < ns) local += sample_entries(cu, s, n, m);
  }
  tmp[t] = local;
  __syncthreads();
  for (int off = 1; off < kThreads; off *= 2) {  // inclusive scan
    const int v = tmp[t] + (t >= off ? tmp[t - off] : 0);
    __syncthreads();
    tmp[t] = v;
    __syncthreads();
  }
  int run = tmp[t] - local;
  for (int u = 0; u < per; ++u) {
    const int s = s0 + u;
    if (s < ns) {
      E[s] = run;
      run += sample_entries(cu, s, n, m);
    }
  }
  if (t == kThreads - 1) E[ns] = tmp[t];
  __syncthreads();
}
// the sample holding packed entry e: the last s with E[s] <= e (a sample without entries
// shares its E with the next one and is skipped)
__device__ __forceinline__ int sample_of(const int* E, int ns, int e) {
  int lo = 0, hi = ns;  // E[lo] <= e < E[hi] once e < E[ns]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (E[mid] <= e) lo = mid;
    else hi = mid;
  }
  return lo;
}

// online per-channel softmax accumulation of one token row (8 channels)
__device__ __forceinline__ void accum8(float* mx, float* den, float* acc, const float* z, const float* cv) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float mn = fmaxf(mx[e], z[e]);
    float a = exp2f((mx[e] - mn) * kLog2e);
    float p = exp2f((z[e] - mn) * kLog2e);
    den[e] = den[e] * a + p;
    acc[e] = acc[e] * a + p * cv[e];
    mx[e] = mn;
  }
}

// x_hat[row, cc0 .. cc0 + kCB) . W[cc0 .. cc0 + kCB, d] added to acc (4 channels per LDS read)
template <int kCB>
__device__ __forceinline__ void project_row(const float* xs, int c, int row, int cc0, const float (&w)[kCB],
                                            float& acc) {
  float a = acc;
#pragma unroll
  for (int q = 0; q < kCB; q += 4) {
    const float4 x4 = *reinterpret_cast<const float4*>(&xs[row * c + cc0 + q]);
    a += x4.x * w[q];
    a += x4.y * w[q + 1];
    a += x4.z * w[q + 2];
    a += x4.w * w[q + 3];
  }
  acc = a;
}

// One thread's share of the indexer-K projection: sum over channels [c_lo, c_lo + span) of
// x_hat[row, ch] * W_ik[ch, d] for the rows below nrows (in chunks of 8; a chunk is uniform
// over the workgroup).  W is read kCB channels at a time, the next block's loads issued
// before the current block is used, so one L2 round trip covers a whole block.
template <typename T, int kCB, int kDIc>
__device__ __forceinline__ void project_part(const float* xs, const T* __restrict__ w_ik, int c, int c_lo,
                                             int span, int d, int nrows, float (&part_sum)[kRowsPerWG]) {
  const int nblk = span / kCB;
  float wcur[kCB], wnxt[kCB];
#pragma unroll
  for (int u = 0; u < kCB; ++u) wcur[u] = Ld<T>::scalar(w_ik + (size_t)(c_lo + u) * kDIc + d);
  for (int blk = 0; blk < nblk; ++blk) {
    const int cc0 = c_lo + kCB * blk;
    // the next block (the last iteration reloads its own block: same load count every trip)
    const int cn = blk + 1 < nblk ? cc0 + kCB : cc0;
#pragma unroll
    for (int u = 0; u < kCB; ++u) wnxt[u] = Ld<T>::scalar(w_ik + (size_t)(cn + u) * kDIc + d);
#pragma unroll
    for (int rc = 0; rc < kRowsPerWG; rc += 8) {
      // a full chunk of 8 rows runs unguarded; a partial one (a decode append has a single
      // row) skips its missing rows.  Both conditions are uniform over the workgroup.
      if (rc + 8 <= nrows) {
#pragma unroll
        for (int r = 0; r < 8; ++r) project_row(xs, c, rc + r, cc0, wcur, part_sum[rc + r]);
      } else if (rc < nrows) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if (rc + r < nrows) project_row(xs, c, rc + r, cc0, wcur, part_sum[rc + r]);
      }
    }
#pragma unroll
    for (int u = 0; u < kCB; ++u) wcur[u] = wnxt[u];
  }
}

template <typename T, int G, int kDI>
__global__ void __launch_bounds__(kThreads) compress_kernel(
    int n, int c, int m, int overlap, const T* __restrict__ ca, const T* __restrict__ za,
    const T* __restrict__ cb, const T* __restrict__ zb, const T* __restrict__ cb0,
    const T* __restrict__ zb0, const float* __restrict__ ba,
    const float* __restrict__ bb, const int32_t* __restrict__ pos0, int norm, float eps,
    int rope_dims, RopeFreq rope, T* __restrict__ out, int64_t out_bstride, int64_t out_cap,
    const T* __restrict__ w_ik, int d_index, T* __restrict__ out_ik, int64_t out_ik_bstride,
    int64_t ik_cap, const int32_t* __restrict__ dst_row, uint8_t* __restrict__ out_codes,
    uint8_t* __restrict__ out_scales, uint8_t* __restrict__ ik_codes, uint8_t* __restrict__ ik_scales,
    int64_t q_rows, const int32_t* __restrict__ cu_seqlens, int n_samples, int e_off,
    int32_t* __restrict__ out_cu_entries) {
  constexpr bool kProj = kDI > 0;
  extern __shared__ float xs[];  // [kRowsPerWG][c] pre-RoPE normalised entries (kProj only)
  const int b = blockIdx.y;
  // packed samples (B = 1): per-sample entry offsets in LDS after the projection's space
  int* E = reinterpret_cast<int*>(xs + e_off);
  int n_ent = n / m;
  if (cu_seqlens) {
    sample_entry_offsets(cu_seqlens, n_samples, n, m, E, E + n_samples + 1);
    n_ent = E[n_samples];
    if (out_cu_entries && blockIdx.x == 0)
      for (int s = threadIdx.x; s <= n_samples; s += kThreads) out_cu_entries[s] = E[s];
  }
  const int row0 = blockIdx.x * kRowsPerWG;
  const int lane_in_row = threadIdx.x % G;
  const int row_slot = threadIdx.x / G;
  constexpr int kRowsPerPass = kThreads / G;
  const int ch = lane_in_row * 8;
  const size_t seq_off = (size_t)b * n * c;
  const int64_t dst0 = dst_row ? (int64_t)dst_row[b] : 0;  // output row of entry 0

  for (int lr = row_slot; lr < kRowsPerWG; lr += kRowsPerPass) {
    const int i = row0 + lr;
    if (i >= n_ent) break;
    // entry i pools tokens tok0 .. tok0 + m - 1 of the stream; il is its block within its
    // sequence (a sample of a packed stream restarts at block 0: positions from 0, no history)
    int il = i, sidx = b;
    int64_t tok0 = (int64_t)m * i;
    if (cu_seqlens) {
      sidx = sample_of(E, n_samples, i);
      il = i - E[sidx];
      int lo, len;
      sample_span(cu_seqlens, sidx, n, &lo, &len);
      tok0 = (int64_t)lo + (int64_t)m * il;
    }
    float mx[8], den[8], acc[8], z[8], cv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mx[e] = -INFINITY; den[e] = 0.f; acc[e] = 0.f; }
    for (int j = 0; j < m; ++j) {
      const size_t off = seq_off + (size_t)(tok0 + j) * c + ch;
      Ld<T>::load8(za + off, z);
      Ld<T>::load8(ca + off, cv);
      if (ba) {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] += ba[j * c + ch + e];
      }
      accum8(mx, den, acc, z, cv);
    }
    // history: the previous block's b-branch rows; entry 0 takes them from cb0 / zb0 when
    // given, else it has none (its -inf logits carry zero weight)
    if (overlap && (il > 0 || cb0)) {
      const T* hc = il > 0 ? cb + seq_off + (size_t)(tok0 - m) * c : cb0 + (size_t)b * m * c;
      const T* hz = il > 0 ? zb + seq_off + (size_t)(tok0 - m) * c : zb0 + (size_t)b * m * c;
      for (int j = 0; j < m; ++j) {
        const size_t off = (size_t)j * c + ch;
        Ld<T>::load8(hz + off, z);
        Ld<T>::load8(hc + off, cv);
        if (bb) {
#pragma unroll
          for (int e = 0; e < 8; ++e) z[e] += bb[j * c + ch + e];
        }
        accum8(mx, den, acc, z, cv);
      }
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = acc[e] / den[e];
    if (norm) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
      ss = group_sum<G>(ss);
      const float inv = fast_rsqrt(ss / (float)c + eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= inv;
    }
    if (kProj) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[lr * c + ch + e] = y[e];
    }
    if (rope_dims > 0 && ch + 8 > c - rope_dims) {
      const double pos = (double)((pos0 ? pos0[sidx] : 0)) + (double)m * (double)il;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int cc = ch + e;
        if (cc >= c - rope_dims) {
          float cs, sn;
          rope_cs(pos, rope.f[(cc - (c - rope_dims)) / 2], &cs, &sn);
          const float x0 = y[e], x1 = y[e + 1];
          y[e] = x0 * cs - x1 * sn;
          y[e + 1] = x0 * sn + x1 * cs;
        }
      }
    }
    const int64_t r_out = dst0 + i;
    if (out && r_out >= 0 && r_out < out_cap) Ld<T>::store8(out + (size_t)b * out_bstride + (size_t)r_out * c + ch, y);
    if (out_codes) {
      // FP4 entry: 16-channel groups are lane pairs of the row
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(y[e]));
      am = fmaxf(am, dpp<kDppXor1>(am));
      const int sb = e4m3_scale_byte(am);
      const float sc = e4m3_value(sb);
      uint32_t word = 0;
      if (sc > 0.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) word |= e2m1_code(y[e], sc) << (4 * e);
      }
      if (r_out >= 0 && r_out < q_rows) {
        const size_t qr = (size_t)b * q_rows + r_out;
        *reinterpret_cast<uint32_t*>(out_codes + qr * (c / 2) + ch / 2) = word;
        if ((lane_in_row & 1) == 0) out_scales[qr * (c / 16) + ch / 16] = (uint8_t)sb;
      }
    }
  }

  if (kProj) {
    __syncthreads();
    // K_I[row, d] = sum_c x_hat[row, c] * W_ik[c, d].  Thread (d, part): the channel range
    // of its part, rows in chunks of 8 (4 channels per LDS read, W loads shared by the
    // chunk's rows); the parts' partial sums then meet in LDS and are added in part order.
    constexpr int kDIc = kProj ? kDI : 128;  // placeholder width when there is no projection
    constexpr int kParts = kThreads / kDIc;
    const int d = threadIdx.x % kDIc;
    const int part = threadIdx.x / kDIc;
    const int nrows = min(kRowsPerWG, n_ent - row0);
    const int span = c / kParts;  // channels per part
    const int c_lo = part * span;
    float part_sum[kRowsPerWG];
#pragma unroll
    for (int r = 0; r < kRowsPerWG; ++r) part_sum[r] = 0.f;
    if (span % 32 == 0)
      project_part<T, 32, kDIc>(xs, w_ik, c, c_lo, span, d, nrows, part_sum);
    else
      project_part<T, 4, kDIc>(xs, w_ik, c, c_lo, span, d, nrows, part_sum);
    __syncthreads();  // every part has read xs: its space takes the partial sums
    float* ps = xs;   // [kParts][kRowsPerWG][kDIc]
#pragma unroll
    for (int r = 0; r < kRowsPerWG; ++r) ps[(part * kRowsPerWG + r) * kDIc + d] = part_sum[r];
    __syncthreads();
    constexpr int kRowsPerPart = kRowsPerWG / kParts;
#pragma unroll
    for (int rr = 0; rr < kRowsPerPart; ++rr) {
      const int r = rr * kParts + part;
      float kv = 0.f;
#pragma unroll
      for (int p = 0; p < kParts; ++p) kv += ps[(p * kRowsPerWG + r) * kDIc + d];
      const int i = row0 + r;
      const int64_t r_out = dst0 + i;
      if (out_ik && i < n_ent && r_out >= 0 && r_out < ik_cap)
        Ld<T>::store1(out_ik + (size_t)b * out_ik_bstride + (size_t)r_out * kDIc + d, kv);
      if (ik_codes) {
        // MXFP4: a 32-value group is an aligned half of the wave (d = lane % 32 + 32 j, one
        // row per half); neighbouring lanes' codes are gathered so each even lane stores one
        // byte
        const float am = max32(fabsf(kv));
        const int e = am > 0.f ? mx_exponent(am) : 0;
        const uint32_t code = am > 0.f ? e2m1_code(__builtin_amdgcn_ldexpf(kv, -e), 1.0f) : 0u;
        const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)code, kDppXor1, 0xF, 0xF, false);
        if (i < n_ent && r_out >= 0 && r_out < q_rows) {
          const size_t qr = (size_t)b * q_rows + r_out;
          if ((d & 1) == 0) ik_codes[qr * (kDIc / 2) + d / 2] = (uint8_t)(code | (hi << 4));
          if ((d & 31) == 0) ik_scales[qr * (kDIc / 32) + d / 32] = (uint8_t)(e + 127);
        }
      }
    }
  }
}

template <typename T, int G, int kDI>
hipError_t launch_t(const csa2_compress_desc& d, hipStream_t s) {
  const int n_ent = d.n / d.m;  // packed samples: an upper bound of their entries
  dim3 grid(std::max((n_ent + kRowsPerWG - 1) / kRowsPerWG, d.cu_seqlens ? 1 : 0), d.B);
  const int64_t ob = d.out_batch_stride ? d.out_batch_stride : (int64_t)n_ent * d.c;
  const int64_t oib = d.out_ik_batch_stride ? d.out_ik_batch_stride : (int64_t)n_ent * d.d_index;
  const int64_t out_cap = ob / d.c, ik_cap = d.d_index ? oib / d.d_index : 0;
  const int64_t q_rows = d.q_rows ? d.q_rows : (int64_t)n_ent;
  // pre-RoPE entries, then (same space) the partial sums of the projection; packed samples
  // add their entry offsets and a scan buffer after it
  const size_t proj_floats = kDI > 0 ? std::max((size_t)kRowsPerWG * d.c, (size_t)kThreads * kRowsPerWG) : 0;
  const size_t lds = (proj_floats + (d.cu_seqlens ? (size_t)d.n_samples + 1 + kThreads : 0)) * sizeof(float);
  RopeFreq rope;
  rope_freq_host(&rope, d.rope_dims, d.rope_theta);
  hipLaunchKernelGGL((compress_kernel<T, G, kDI>), grid, dim3(kThreads), lds, s, d.n, d.c, d.m,
                     d.overlap, (const T*)d.ca, (const T*)d.za, (const T*)d.cb, (const T*)d.zb,
                     (const T*)d.cb0, (const T*)d.zb0, d.ba,
                     d.bb, d.pos0, d.norm, d.eps, d.rope_dims, rope, (T*)d.out, ob, out_cap,
                     (const T*)d.w_ik, d.d_index, (T*)d.out_ik, oib, ik_cap, d.dst_row,
                     d.out_codes, d.out_scales, d.w_ik ? d.ik_codes : nullptr, d.ik_scales, q_rows,
                     d.cu_seqlens, d.n_samples, (int)proj_floats, d.out_cu_entries);
  return hipGetLastError();
}

template <typename T, int G>
hipError_t launch_g(const csa2_compress_desc& d, hipStream_t s) {
  if (!d.w_ik) return launch_t<T, G, 0>(d, s);
  switch (d.d_index) {
    case 32: return launch_t<T, G, 32>(d, s);
    case 64: return launch_t<T, G, 64>(d, s);
    case 128: return launch_t<T, G, 128>(d, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_dt(const csa2_compress_desc& d, hipStream_t s) {
  switch (d.c / 8) {
    case 1: return launch_g<T, 1>(d, s);
    case 2: return launch_g<T, 2>(d, s);
    case 4: return launch_g<T, 4>(d, s);
    case 8: return launch_g<T, 8>(d, s);
    case 16: return launch_g<T, 16>(d, s);
    case 32: return launch_g<T, 32>(d, s);
    case 64: return launch_g<T, 64>(d, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_compress(const csa2_compress_desc& d, hipStream_t s) {
  if (d.n / d.m == 0 && !(d.cu_seqlens && d.out_cu_entries)) return hipSuccess;
  // every pointer a kernel dereferences must be set
  if (!d.ca || !d.za || (!d.out && !d.out_codes) || (d.overlap && (!d.cb || !d.zb)) ||
      (d.w_ik && !d.out_ik && !d.ik_codes) || (!d.out_codes != !d.out_scales) ||
      (!d.ik_codes != !d.ik_scales) || (d.out_codes && d.c % 16 != 0) || (!d.cb0 != !d.zb0) ||
      (d.cu_seqlens && (d.B != 1 || d.n_samples < 1 || d.n_samples > kMaxSamples || d.cb0)))
    return hipErrorInvalidValue;
  ScopedProf p(s, "compress");
  return d.dtype == CSA2_F32 ? launch_dt<float>(d, s) : launch_dt<uint16_t>(d, s);
}

}  // namespace csa2

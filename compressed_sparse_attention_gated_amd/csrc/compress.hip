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

template <typename T, int G, int kDI>
__global__ void __launch_bounds__(kThreads) compress_kernel(
    int n, int c, int m, int overlap, const T* __restrict__ ca, const T* __restrict__ za,
    const T* __restrict__ cb, const T* __restrict__ zb, const float* __restrict__ ba,
    const float* __restrict__ bb, const int32_t* __restrict__ pos0, int norm, float eps,
    int rope_dims, RopeFreq rope, T* __restrict__ out, int64_t out_bstride,
    const T* __restrict__ w_ik, int d_index, T* __restrict__ out_ik, int64_t out_ik_bstride) {
  constexpr bool kProj = kDI > 0;
  extern __shared__ float xs[];  // [kRowsPerWG][c] pre-RoPE normalised entries (kProj only)
  const int n_ent = n / m;
  const int b = blockIdx.y;
  const int row0 = blockIdx.x * kRowsPerWG;
  const int lane_in_row = threadIdx.x % G;
  const int row_slot = threadIdx.x / G;
  constexpr int kRowsPerPass = kThreads / G;
  const int ch = lane_in_row * 8;
  const size_t seq_off = (size_t)b * n * c;

  for (int lr = row_slot; lr < kRowsPerWG; lr += kRowsPerPass) {
    const int i = row0 + lr;
    if (i >= n_ent) break;
    float mx[8], den[8], acc[8], z[8], cv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mx[e] = -INFINITY; den[e] = 0.f; acc[e] = 0.f; }
    for (int j = 0; j < m; ++j) {
      const size_t off = seq_off + (size_t)(m * i + j) * c + ch;
      Ld<T>::load8(za + off, z);
      Ld<T>::load8(ca + off, cv);
      if (ba) {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] += ba[j * c + ch + e];
      }
      accum8(mx, den, acc, z, cv);
    }
    if (overlap && i > 0) {  // entry 0 has no history: its -inf logits carry zero weight
      for (int j = 0; j < m; ++j) {
        const size_t off = seq_off + (size_t)(m * (i - 1) + j) * c + ch;
        Ld<T>::load8(zb + off, z);
        Ld<T>::load8(cb + off, cv);
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
      const double pos = (double)((pos0 ? pos0[b] : 0)) + (double)m * (double)i;
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
    Ld<T>::store8(out + (size_t)b * out_bstride + (size_t)i * c + ch, y);
  }

  if (kProj) {
    __syncthreads();
    // K_I[row, d] = sum_c x_hat[row, c] * W_ik[c, d]; thread -> (d, row group)
    constexpr int kDIc = kProj ? kDI : 128;  // placeholder width when there is no projection
    constexpr int kGroups = kThreads / kDIc;
    constexpr int kRowsPerGroup = kRowsPerWG / kGroups;
    const int d = threadIdx.x % kDIc;
    const int rg = threadIdx.x / kDIc;
    float accp[kRowsPerGroup];
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) accp[r] = 0.f;
    for (int cc = 0; cc < c; ++cc) {
      const float wv = Ld<T>::scalar(w_ik + (size_t)cc * kDIc + d);
#pragma unroll
      for (int r = 0; r < kRowsPerGroup; ++r) accp[r] += xs[(rg * kRowsPerGroup + r) * c + cc] * wv;
    }
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) {
      const int i = row0 + rg * kRowsPerGroup + r;
      if (i < n_ent) Ld<T>::store1(out_ik + (size_t)b * out_ik_bstride + (size_t)i * kDIc + d, accp[r]);
    }
  }
}

template <typename T, int G, int kDI>
hipError_t launch_t(const csa2_compress_desc& d, hipStream_t s) {
  const int n_ent = d.n / d.m;
  dim3 grid((n_ent + kRowsPerWG - 1) / kRowsPerWG, d.B);
  const int64_t ob = d.out_batch_stride ? d.out_batch_stride : (int64_t)n_ent * d.c;
  const int64_t oib = d.out_ik_batch_stride ? d.out_ik_batch_stride : (int64_t)n_ent * d.d_index;
  const size_t lds = kDI > 0 ? (size_t)kRowsPerWG * d.c * sizeof(float) : 0;
  RopeFreq rope;
  rope_freq_host(&rope, d.rope_dims, d.rope_theta);
  hipLaunchKernelGGL((compress_kernel<T, G, kDI>), grid, dim3(kThreads), lds, s, d.n, d.c, d.m,
                     d.overlap, (const T*)d.ca, (const T*)d.za, (const T*)d.cb, (const T*)d.zb, d.ba,
                     d.bb, d.pos0, d.norm, d.eps, d.rope_dims, rope, (T*)d.out, ob,
                     (const T*)d.w_ik, d.d_index, (T*)d.out_ik, oib);
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
  if (d.n / d.m == 0) return hipSuccess;
  // every pointer a kernel dereferences must be set
  if (!d.ca || !d.za || !d.out || (d.overlap && (!d.cb || !d.zb)) || (d.w_ik && !d.out_ik))
    return hipErrorInvalidValue;
  ScopedProf p(s, "compress");
  return d.dtype == CSA2_F32 ? launch_dt<float>(d, s) : launch_dt<uint16_t>(d, s);
}

}  // namespace csa2

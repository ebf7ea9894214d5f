// Sparse shared-KV MQA over the selected entries plus the sliding window
// ([DSA-to-CSA notes] eq. (18)-(19) and "Shared-KV MQA": every selected entry is both key
// and value, the query heads are RMS-normalised and rotated on the last r dims, the output's
// last r dims are rotated back by the query position; eq. (27): one value-less sink logit
// per head in the softmax denominator; [CSA2 column] "保留了 CSA 的骨架": the selected
// entries are joined by the latest 128 uncompressed rows of the layer).
//
// attn_mfma (bf16 queries, 64 heads per workgroup, c = 512, bf16 or FP4 rows):
//   One workgroup = one query x 64 heads x a contiguous range of row slots (a split): 8
//   waves in two halves of 32 heads that share every row tile in LDS, so each selected row
//   is read once per query.  Rows are gathered a tile at a time into LDS (64 rows for bf16,
//   32 for FP4, whose larger register set spills at 64; FP4 rows are dequantised on the way:
//   E2M1 x E4M3 is exact in bf16), one tile in flight in registers; the workgroup barriers
//   order LDS only, so the next tile's loads stay in flight across them.  Wave (half, hq,
//   mr) computes the S^T blocks of rows 32*kk + 16*mr.. x heads 32*half + 16*hq.. on
//   v_mfma_f32_16x16x32_bf16 (q_hat in registers; two independent accumulators in a 64-row
//   tile); the C layout of S^T gives each lane one head and 4 rows per block, written to LDS
//   in the A-operand order of P for the PV product.  For PV each wave owns 128 output
//   channels of its half's 32 heads; the V operand (rows along K) is read with the gfx950
//   LDS transpose read ds_read_b64_tr_b16 from the same row-major tile that fed S^T (shared
//   K = V, one copy in LDS).  The row pitch is padded by 32 bytes, which keeps the
//   transposing PV reads free of bank conflicts (see kPitch).  Softmax in fp32 with exp2 (scale folded into q_hat) against a
//   fixed per-head reference (see kOverflow).  With several splits per query each split's
//   output (normalised by its own sum, bf16) and (max, sum) go to a workspace in 32-head
//   units and attn_combine merges them in a fixed order.
//
// attn_simple: any head count / width / dtype; one wave per (query, head), fp32 math.

#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

// ------------------------------------------------------------------ shared row bookkeeping
struct AttnDev {
  int B, T, H, c, k, N, rope_dims, q_norm, Lw, n_win, splits, tiles_per_split, n_hg;
  int dense_m;  // > 0: the index slots are entries 0 .. N-1, visible up to min(N, t / dense_m)
  float rope_theta, eps, scale_log2;  // scale * log2(e)
  int q_f32, kv_kind;                 // kv_kind: 0 = same as q, 1 = FP4
  const void* q;
  const int32_t* q_pos;
  const void* kv;
  const uint8_t* kv_codes;
  const uint8_t* kv_scales;
  const int32_t* idx;
  const void* win;
  const int32_t* win_pos0;
  const int32_t* win_row0;  // [rows] or null: packed samples, the window row of the sample's position 0
  const float* sink;
  void* out;
  float* out_mass;
  uint16_t* part_o;  // [rows][n_hg][splits][32][c] bf16: each split's output / its own sum
  float* part_ml;    // [rows][n_hg][splits][2][32]: each split's (reference m, sum l)
  RopeFreq rope;   // theta^(-2u/r)
};

struct WinRange {
  int lo_row, cnt;
};
// entries of the index slots visible to a query at position t_pos: all N with an index list
// (its ids say which), the completed blocks' entries in dense mode
__device__ __forceinline__ int slot_limit(const AttnDev& a, int t_pos) {
  return a.dense_m > 0 ? min(a.N, max(t_pos, 0) / a.dense_m) : a.N;
}
__device__ __forceinline__ WinRange window_of_p0(const AttnDev& a, int p0, int t_pos) {
  WinRange w{0, 0};
  if (!a.win || a.n_win <= 0) return w;
  const int lo = max(t_pos - a.n_win + 1, p0);
  const int hi = min(t_pos, p0 + a.Lw - 1);
  if (hi >= lo) { w.lo_row = lo - p0; w.cnt = hi - lo + 1; }
  return w;
}
// The window rows of query `row` (sequence b, position t_pos).  Packed samples: positions
// [max(0, t - W + 1), t] of the query's own sample, at rows win_row0 + position.
__device__ __forceinline__ WinRange window_of(const AttnDev& a, int b, int row, int t_pos) {
  if (a.win && a.n_win > 0 && a.win_row0) {
    WinRange w{0, 0};
    const int r0 = a.win_row0[row];
    const int lo = max(r0 + max(t_pos - a.n_win + 1, 0), 0);
    const int hi = min(r0 + t_pos, a.Lw - 1);
    if (t_pos >= 0 && hi >= lo) { w.lo_row = lo; w.cnt = hi - lo + 1; }
    return w;
  }
  return window_of_p0(a, (a.win && a.n_win > 0) ? a.win_pos0[b] : 0, t_pos);
}

// ------------------------------------------------------------------ attn_simple
template <typename TQ>
__device__ __forceinline__ float ldq(const TQ* p);
template <>
__device__ __forceinline__ float ldq<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldq<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }
template <typename TQ>
__device__ __forceinline__ void stq(TQ* p, float v);
template <>
__device__ __forceinline__ void stq<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void stq<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }

constexpr int kSimpleMaxPerLane = 8;  // c <= 512

template <typename TQ>
__global__ void __launch_bounds__(64) attn_simple(AttnDev a) {
  const int qh = blockIdx.x;  // (row, head)
  const int row = qh / a.H, h = qh % a.H;
  const int b = row / a.T;
  const int lane = threadIdx.x;
  const int c = a.c;
  const int t_pos = a.q_pos[row];
  const TQ* q = (const TQ*)a.q + ((size_t)row * a.H + h) * c;
  float qv[kSimpleMaxPerLane];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) {
    const int ch = lane + 64 * j;
    qv[j] = ch < c ? ldq<TQ>(q + ch) : 0.f;
    ss += qv[j] * qv[j];
  }
  if (a.q_norm) {
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)c + a.eps);
#pragma unroll
    for (int j = 0; j < kSimpleMaxPerLane; ++j) qv[j] *= inv;
  }
  // rope on channels >= c - r: pair (ch, ch^1) sits in lanes (lane, lane^1)
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) {
    const int ch = lane + 64 * j;
    const float other = dpp<kDppXor1>(qv[j]);
    if (a.rope_dims > 0 && ch < c && ch >= c - a.rope_dims) {
      float cs, sn;
      rope_cs((double)t_pos, a.rope.f[(ch - (c - a.rope_dims)) / 2], &cs, &sn);
      qv[j] = (ch & 1) ? (other * sn + qv[j] * cs) : (qv[j] * cs - other * sn);
    }
  }
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) qv[j] *= a.scale_log2;

  const WinRange wr = window_of(a, b, row, t_pos);
  const int R = a.k + wr.cnt;
  const int lim = slot_limit(a, t_pos);
  float m_run = -INFINITY, l_run = 0.f;
  float o[kSimpleMaxPerLane];
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) o[j] = 0.f;
  for (int s = 0; s < R; ++s) {
    float rv[kSimpleMaxPerLane];
    bool valid = true;
    if (s < a.k) {
      const int e = a.dense_m > 0 ? s : a.idx[(size_t)row * a.k + s];
      valid = e >= 0 && e < lim;
      if (!valid) continue;
      if (a.kv_kind == 1) {
        const uint8_t* cp = a.kv_codes + ((size_t)b * a.N + e) * (c / 2);
        const uint8_t* sp = a.kv_scales + ((size_t)b * a.N + e) * (c / 16);
#pragma unroll
        for (int j = 0; j < kSimpleMaxPerLane; ++j) {
          const int ch = lane + 64 * j;
          rv[j] = ch < c ? e2m1_to_f32((cp[ch / 2] >> (4 * (ch & 1))) & 15u) * e4m3_to_f32(sp[ch / 16]) : 0.f;
        }
      } else {
        const TQ* rp = (const TQ*)a.kv + ((size_t)b * a.N + e) * c;
#pragma unroll
        for (int j = 0; j < kSimpleMaxPerLane; ++j) {
          const int ch = lane + 64 * j;
          rv[j] = ch < c ? ldq<TQ>(rp + ch) : 0.f;
        }
      }
    } else {
      const TQ* rp = (const TQ*)a.win + ((size_t)b * a.Lw + wr.lo_row + (s - a.k)) * c;
#pragma unroll
      for (int j = 0; j < kSimpleMaxPerLane; ++j) {
        const int ch = lane + 64 * j;
        rv[j] = ch < c ? ldq<TQ>(rp + ch) : 0.f;
      }
    }
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < kSimpleMaxPerLane; ++j) d += qv[j] * rv[j];
    d = wave_sum(d);
    const float m_new = fmaxf(m_run, d);
    const float alpha = exp2f(m_run - m_new);  // m_run = -inf -> 0
    const float p = exp2f(d - m_new);
    l_run = l_run * alpha + p;
#pragma unroll
    for (int j = 0; j < kSimpleMaxPerLane; ++j) o[j] = o[j] * alpha + p * rv[j];
    m_run = m_new;
  }
  float denom = l_run;
  if (a.sink && l_run > 0.f) denom += exp2f(a.sink[h] * kLog2e - m_run);
  const float inv = l_run > 0.f ? 1.0f / denom : 0.f;
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) o[j] *= inv;
  // inverse rotation of the output's last r channels by the query position
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) {
    const int ch = lane + 64 * j;
    const float other = dpp<kDppXor1>(o[j]);
    if (a.rope_dims > 0 && ch < c && ch >= c - a.rope_dims) {
      float cs, sn;
      rope_cs(-(double)t_pos, a.rope.f[(ch - (c - a.rope_dims)) / 2], &cs, &sn);
      o[j] = (ch & 1) ? (other * sn + o[j] * cs) : (o[j] * cs - other * sn);
    }
  }
  TQ* op = (TQ*)a.out + ((size_t)row * a.H + h) * c;
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) {
    const int ch = lane + 64 * j;
    if (ch < c) stq<TQ>(op + ch, o[j]);
  }
  if (a.out_mass && lane == 0) a.out_mass[(size_t)row * a.H + h] = l_run > 0.f ? l_run * inv : 0.f;
}

// ------------------------------------------------------------------ attn_mfma
constexpr int kC = 512;           // channels
constexpr int kHG = 32;           // heads per split-partial unit (one half of a workgroup)
// rows per tile: 64 for bf16 rows (fewer barriers and exchanges per row); 32 for FP4 rows,
// whose larger register prefetch set (codes, scales and bf16 window rows) spills at 64
template <bool kFP4>
constexpr int kTileOf = kFP4 ? 32 : 64;
constexpr int kRowBytes = kC * 2;
constexpr int kThreadsM = 512;    // 8 waves: two halves of 4, one per 32 heads
constexpr int kHW = 2 * kHG;       // heads per workgroup
constexpr int kWaves = kThreadsM / 64;
template <int kT>
constexpr int kPrefRows = kT / kWaves;          // bf16 rows each wave loads per tile
template <int kT>
constexpr int kFp4Per = kT * 16 / kThreadsM;    // FP4 16-byte code chunks per thread per tile

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS row pitch: 1024 B of bf16 channels + 32 B, a stride of 8 of the 64 banks per row, so
// one transposing PV read (32 lanes: 8 rows x 32 B) covers the banks once.  Every offset
// inside a tile is a compile-time immediate.  (16 B of padding keeps the S^T A-operand rows
// apart instead, but leaves the PV reads two-way conflicted: 8-9 % slower on long rows.)
constexpr int kPitch = kRowBytes + 32;
constexpr int kMaxSplitRows = 1024;   // row slots per split (staged in LDS)
// Softmax reference: each head fixes the max of its first valid tile as the reference m
// and keeps it; the final normalisation divides by a sum taken with the same reference,
// so the result is the exact softmax for any m, and the accumulators are never rescaled.
// Terms are 2^(z - m) <= 2^kOverflow; if a later tile exceeds m by more than that, the
// split starts again with the larger reference (never for normalised inputs, where
// |z| <= sqrt(c) * log2(e)).
constexpr float kOverflow = 60.0f;

template <int kT>
struct MfmaSmem {
  static constexpr int kPPitch = kT + 8;  // P rows (bf16), padded likewise
  // two row tiles; the same bytes also stage q_hat ([32 heads][kPitch]) before the loop
  // and the bf16 output tile ([32][512]) after it
  alignas(16) uint8_t tile[2][kT * kPitch];
  alignas(16) uint16_t pbuf[kHW][kPPitch];  // P in PV A-operand order (bf16)
  float wmax[2][kHW];                       // per row half: tile max per head (first valid tile)
  float omax[2][kHW];                       // per row half: tile max per head (overflow check)
  float lpart[2][kHW];                      // per row half: sum of p per head
  float mfin[kHW];
  float rope_c[64], rope_s[64];             // cos/sin of the query position, per frequency
  alignas(16) int ovf[kWaves];              // per wave: a head overflowed its reference
  int src[kMaxSplitRows];                   // per slot: >= 0 kv entry id, -2-w window row w, -1 empty
};
static_assert(sizeof(MfmaSmem<64>) <= 160 * 1024, "LDS of one workgroup (one per CU)");
static_assert(2 * 32 * kPitch >= kHW * kPitch, "q_hat of the workgroup's heads fits the two row tiles");

// registers for one tile in flight.  bf16 rows: wave w owns rows w, w+8, .., w+24 and
// lane l carries their 16-byte chunk l.  FP4 rows: thread q carries code chunk q%16 of row
// q/16 and the two E4M3 scales of its 32 channels.
template <bool kFP4, int kT = kTileOf<kFP4>>
struct Prefetch {
  uint4 v[kPrefRows<kT>];
  uint4 fc[kFP4 ? kFp4Per<kT> : 1];
  uint32_t fs[kFP4 ? kFp4Per<kT> : 1];
};

// Slot -> row source for this split's slots [slot0, slot0 + n): index slot s < k holds its
// entry id (-1 if empty or out of range), slot k + w window row lo_row + w as -2 - row,
// slots past R are empty.  The index slots do not depend on the query position, so their
// ids are loaded first (ids_of_split) and only combined with the window here.
constexpr int kSlotsPerThread = kMaxSplitRows / kThreadsM;
static_assert(kMaxSplitRows == kSlotsPerThread * kThreadsM, "slot ids per thread");
__device__ __forceinline__ void ids_of_split(const AttnDev& a, int row, int slot0, int n,
                                             int (&ids)[kSlotsPerThread]) {
#pragma unroll
  for (int u = 0; u < kSlotsPerThread; ++u) {
    const int i = threadIdx.x + kThreadsM * u;
    const int s = slot0 + i;
    ids[u] = (i < n && s < a.k) ? (a.dense_m > 0 ? s : a.idx[(size_t)row * a.k + s]) : -1;
  }
}
__device__ __forceinline__ void stage_slots(const AttnDev& a, int slot0, int n, int R, const WinRange& wr,
                                            int lim, const int (&ids)[kSlotsPerThread], int* src) {
#pragma unroll
  for (int u = 0; u < kSlotsPerThread; ++u) {
    const int i = threadIdx.x + kThreadsM * u;
    if (i >= n) break;
    const int s = slot0 + i;
    int v = -1;
    if (s < R) {
      if (s < a.k) v = (ids[u] >= 0 && ids[u] < lim) ? ids[u] : -1;
      else v = -2 - (wr.lo_row + (s - a.k));
    }
    src[i] = v;
  }
}

// Row sources of one sequence, computed once per workgroup: the kernel arguments they come
// from would otherwise be reloaded after every barrier (its memory clobber) for every row.
struct RowBases {
  const uint16_t* kv;       // bf16 cache rows of the sequence
  const uint16_t* win;      // window rows of the sequence
  const uint8_t* codes;     // FP4 cache rows: codes
  const uint8_t* scales;    //                 and E4M3 scales
};
__device__ __forceinline__ RowBases row_bases(const AttnDev& a, int b) {
  RowBases r;
  r.kv = (const uint16_t*)a.kv + (size_t)b * a.N * kC;
  r.win = (const uint16_t*)a.win + (size_t)b * a.Lw * kC;
  r.codes = a.kv_codes + (size_t)b * a.N * (kC / 2);
  r.scales = a.kv_scales + (size_t)b * a.N * (kC / 16);
  return r;
}

template <bool kFP4>
__device__ __forceinline__ void fetch_tile(const RowBases& rb, const int* src, Prefetch<kFP4>& pf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kPR = kPrefRows<kTileOf<kFP4>>;
  int srow[kPR];
#pragma unroll
  for (int i = 0; i < kPR; ++i) srow[i] = src[wave + kWaves * i];  // all slot reads first, one wait
#pragma unroll
  for (int i = 0; i < kPR; ++i) {
    const int sr = __builtin_amdgcn_readfirstlane(srow[i]);  // uniform per wave
    const uint16_t* base = nullptr;
    if (sr <= -2) base = rb.win + (size_t)(-2 - sr) * kC;
    else if (!kFP4 && sr >= 0) base = rb.kv + (size_t)sr * kC;
    pf.v[i] = base ? reinterpret_cast<const uint4*>(base)[lane] : make_uint4(0, 0, 0, 0);
  }
  if constexpr (kFP4) {
#pragma unroll
    for (int i = 0; i < kFp4Per<kTileOf<kFP4>>; ++i) {
      const int q = threadIdx.x + kThreadsM * i;
      const int r = q >> 4, part = q & 15;
      const int sr = src[r];
      if (sr >= 0) {
        pf.fc[i] = reinterpret_cast<const uint4*>(rb.codes + (size_t)sr * (kC / 2))[part];
        pf.fs[i] = *reinterpret_cast<const uint16_t*>(rb.scales + (size_t)sr * (kC / 16) + 2 * part);
      } else {
        pf.fc[i] = make_uint4(0, 0, 0, 0);
        pf.fs[i] = 0;
      }
    }
  }
}

template <bool kFP4>
__device__ __forceinline__ void commit_tile(const int* src, const Prefetch<kFP4>& pf, uint8_t* tile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kPrefRows<kTileOf<kFP4>>; ++i) {
    const int r = wave + kWaves * i;
    const int sr = __builtin_amdgcn_readfirstlane(src[r]);
    if (!kFP4 || sr < 0) *reinterpret_cast<uint4*>(tile + r * kPitch + 16 * lane) = pf.v[i];
  }
  if constexpr (kFP4) {
#pragma unroll
    for (int i = 0; i < kFp4Per<kTileOf<kFP4>>; ++i) {
      const int q = threadIdx.x + kThreadsM * i;
      const int r = q >> 4, part = q & 15;
      if (src[r] >= 0) {
        // 32 codes -> channels 32*part .. 32*part+31; scales of groups 2*part, 2*part+1.
        // The hardware's FP4 convert (unit scale) gives each code's E2M1 value, two codes
        // (one byte, low nibble first) per instruction; times the E4M3 scale the product
        // has at most 6 significant bits, so it is exact in fp32 and in bf16.
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const float s0 = e4m3_to_f32(pf.fs[i] & 0xffu), s1 = e4m3_to_f32(pf.fs[i] >> 8);
        const uint32_t words[4] = {pf.fc[i].x, pf.fc[i].y, pf.fc[i].z, pf.fc[i].w};
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          float f[8];
          const float sc = qq < 2 ? s0 : s1;
          const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[qq], 1.0f, 0);
          const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[qq], 1.0f, 1);
          const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[qq], 1.0f, 2);
          const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(words[qq], 1.0f, 3);
          f[0] = v0.x * sc; f[1] = v0.y * sc; f[2] = v1.x * sc; f[3] = v1.y * sc;
          f[4] = v2.x * sc; f[5] = v2.y * sc; f[6] = v3.x * sc; f[7] = v3.y * sc;
          *reinterpret_cast<uint4*>(tile + r * kPitch + 64 * part + 16 * qq) = pack8(f);
        }
      }
    }
  }
}

// cos/sin of t_pos * theta^(-2u/r) for u < r/2, one thread per frequency
__device__ __forceinline__ void stage_rope(const AttnDev& a, int t_pos, float* rc, float* rs) {
  const int u = threadIdx.x;
  if (a.rope_dims > 0 && u < a.rope_dims / 2) rope_cs((double)t_pos, a.rope.f[u], &rc[u], &rs[u]);
}

// Workgroup = one query x 64 heads x one split of its row slots: two halves of 4 waves,
// one per 32 heads, share every row tile in LDS (each row is read once per query).  Wave
// (half, hq, mr): S^T tile rows 16*mr.. x heads 32*half + 16*hq.. of each 32-row tile; for
// PV, wave (half, w4) owns output channels 128*w4 .. 128*w4+127 of its half's 32 heads.
template <bool kFP4>
__global__ void __launch_bounds__(kThreadsM, 1) attn_mfma(AttnDev a) {
  constexpr int kTile = kTileOf<kFP4>;
  constexpr int kKK = kTile / 32;  // 32-row blocks per tile (k steps of PV)
  extern __shared__ __align__(16) uint8_t smem_raw[];
  MfmaSmem<kTile>& sm = *reinterpret_cast<MfmaSmem<kTile>*>(smem_raw);
  const int split = blockIdx.y;
  const int hg = blockIdx.z;
  const int row = blockIdx.x;
  const int b = row / a.T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int half = wave >> 2, w4 = wave & 3;
  const int hq = w4 & 1, mr = w4 >> 1;
  const int tile0 = split * a.tiles_per_split;
  const int rope_lo = kC - a.rope_dims;
  const int head0 = hg * kHW;  // the workgroup's first head
  const RowBases rb = row_bases(a, b);

  // ---- every global load of the prologue at once: the q rows of this wave's 8 heads, the
  // ---- split's index slots, the query position
  uint4 qraw[8];
#pragma unroll
  for (int hh = 0; hh < 8; ++hh)
    qraw[hh] = *reinterpret_cast<const uint4*>((const uint16_t*)a.q + ((size_t)row * a.H + head0 + 8 * wave + hh) * kC + 8 * lane);
  int ids[kSlotsPerThread];
  ids_of_split(a, row, tile0 * kTile, a.tiles_per_split * kTile, ids);
  const int t_pos = a.q_pos[row];
  const WinRange wr = window_of(a, b, row, t_pos);
  const int R = a.k + wr.cnt;
  const int n_tiles = (R + kTile - 1) / kTile;
  const int tile1 = min(tile0 + a.tiles_per_split, n_tiles);
  if (tile0 < tile1) stage_slots(a, tile0 * kTile, (tile1 - tile0) * kTile, R, wr, slot_limit(a, t_pos), ids, sm.src);
  stage_rope(a, t_pos, sm.rope_c, sm.rope_s);
  lds_barrier();
  // rows of the first tile start travelling while q_hat is formed
  Prefetch<kFP4> pf;
  if (tile0 < tile1) fetch_tile<kFP4>(rb, sm.src, pf);

  // ---- q_hat = RoPE_t(RMSNorm(q)) * scale * log2(e) -> LDS (bf16) -> B-operand registers
  uint8_t* qs = sm.tile[0];  // [64 heads][kPitch], across both row tiles
  float qf[8][8];
  float ssq[8];
#pragma unroll
  for (int hh = 0; hh < 8; ++hh) {
    unpack8(qraw[hh], qf[hh]);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += qf[hh][e] * qf[hh][e];
    ssq[hh] = ss;
  }
  if (a.q_norm) {
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) ssq[hh] = wave_sum(ssq[hh]);
  }
  const bool rope_lane = a.rope_dims > 0 && 8 * lane + 8 > rope_lo;
#pragma unroll
  for (int hh = 0; hh < 8; ++hh) {
    float* f = qf[hh];
    const float mul = a.q_norm ? a.scale_log2 * fast_rsqrt(ssq[hh] / (float)kC + a.eps) : a.scale_log2;
    if (rope_lane) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int ch = 8 * lane + e;
        const int u = max(ch - rope_lo, 0) >> 1;
        const float cs = ch >= rope_lo ? sm.rope_c[u] : 1.f, sn = ch >= rope_lo ? sm.rope_s[u] : 0.f;
        const float x0 = f[e], x1 = f[e + 1];
        f[e] = x0 * cs - x1 * sn;
        f[e + 1] = x0 * sn + x1 * cs;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] *= mul;
    *reinterpret_cast<uint4*>(qs + (8 * wave + hh) * kPitch + 16 * lane) = pack8(f);
  }
  lds_barrier();
  bf16x8 qreg[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
    qreg[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qs + (32 * half + 16 * hq + li) * kPitch + 64 * ks + 16 * g));
  lds_barrier();

  // per-lane LDS byte offsets (tile-relative): A operand row 32*kk + 16*mr + li at chunk g
  // (this wave's two 16-row blocks kk = 0, 1); transpose-read source rows 32*kk + 4g + li/4
  // (and +16) at channel 128*w4 + 4*(li%4)
  const int a_off = (16 * mr + li) * kPitch + 16 * g;
  const int t_off0 = (4 * g + (li >> 2)) * kPitch + 8 * (li & 3) + 256 * w4;
  const int t_off1 = t_off0 + 16 * kPitch;
  const int my_head = 32 * half + 16 * hq + li;  // WG-local head of this lane's S^T column

  float m_use = -INFINITY, l_part = 0.f;  // head my_head, rows of half mr (replicated over g)
  // Set once the reference is fixed.  It is decided from the tile's row validity, which is
  // the same for every wave, so the barrier inside that branch is reached by all waves even
  // when a head's scores are NaN (fmaxf drops NaN, which would leave its max at -inf).
  bool ref_set = false;
  f32x4 oacc[2][8];
  for (int pass = 0;; ++pass) {
    if (pass > 0) {  // restart with a larger reference: every wave left the loop together
      lds_barrier();
      fetch_tile<kFP4>(rb, sm.src, pf);
    }
    l_part = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool overflow = false;
    int buf = 0;
    for (int ti = tile0; ti < tile1; ++ti) {
      const int* src = sm.src + (ti - tile0) * kTile;
      commit_tile<kFP4>(src, pf, sm.tile[buf]);
      lds_barrier();
      if (ti + 1 < tile1) fetch_tile<kFP4>(rb, src + kTile, pf);
      // valid rows of this wave's blocks: row 32*kk + 16*mr + r <-> bit 16*kk + r
      const uint32_t vm = (uint32_t)__ballot(lane < 16 * kKK && src[32 * (lane >> 4) + 16 * mr + (lane & 15)] != -1);
      // any valid row in the whole tile: identical in every wave
      const bool tile_any = __ballot(lane < kTile && src[lane] != -1) != 0;

      const uint8_t* tl = sm.tile[buf];
      const lds_u8* tl3 = (const lds_u8*)tl;
      // ---- S^T tile: rows 32*kk + 16*mr.. x heads 16*hq.., two independent accumulators;
      // each block's A reads issued ahead of its MFMAs
      f32x4 sacc[kKK];
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) {
        bf16x8 av[16];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
          av[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(tl + a_off + 32 * kk * kPitch + 64 * ks));
        sacc[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) sacc[kk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ks], qreg[ks], sacc[kk], 0, 0, 0);
      }
      // lane holds head my_head, rows 32*kk + 16*mr + 4*g + j
      bool valid[kKK][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          valid[kk][j] = (vm >> (16 * kk + 4 * g + j)) & 1u;
          if (valid[kk][j]) tmax = fmaxf(tmax, sacc[kk][j]);
        }
      tmax = rows_max(tmax);  // this wave's rows
      // The reference is fixed by the first tile holding a valid row, the max over all
      // of its rows (exchanged between the two waves of a head block).  Validity is per row,
      // the same for every head, so the branch is uniform over the workgroup.  Later tiles
      // only check their own rows against it; the overflow flag is exchanged with P below.
      // A head whose scores are all NaN has no max: it takes 0 (its output is NaN anyway).
      if (!ref_set && tile_any) {
        if (g == 0) sm.wmax[mr][my_head] = tmax;
        lds_barrier();
        tmax = fmaxf(sm.wmax[0][my_head], sm.wmax[1][my_head]);
        m_use = tmax == -INFINITY ? 0.f : tmax;  // O is still 0
        ref_set = true;
      }
      const bool ovf = tmax > m_use + kOverflow;
      if (g == 0) sm.omax[mr][my_head] = tmax;
      float psum = 0.f;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = valid[kk][j] ? exp2f(sacc[kk][j] - m_use) : 0.f;
          psum += p[j];
        }
        // P for head my_head, k-slot 32*kk + 8g + 4*mr + j = row 32*kk + 16*mr + 4g + j
        *reinterpret_cast<uint2*>(&sm.pbuf[my_head][32 * kk + 8 * g + 4 * mr]) =
            make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
      }
      l_part += rows_sum(psum);
      // the vote is taken with every lane active (inside `lane == 0` it would see one head)
      const bool wave_ovf = __ballot(ovf) != 0;
      if (lane == 0) sm.ovf[wave] = wave_ovf;
      lds_barrier();
      const int4 ov0 = *reinterpret_cast<const int4*>(sm.ovf);
      const int4 ov1 = *reinterpret_cast<const int4*>(sm.ovf + 4);
      if (__builtin_amdgcn_readfirstlane(ov0.x | ov0.y | ov0.z | ov0.w | ov1.x | ov1.y | ov1.z | ov1.w)) {
        overflow = true;
        m_use = fmaxf(m_use, fmaxf(sm.omax[0][my_head], sm.omax[1][my_head]));  // whole tile
        break;
      }

      // ---- O[half's heads, 128*w4 .. +128] += P x V, the tile's rows in two k steps of 32
      bf16x8 pa[kKK][2];
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          pa[kk][mt] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.pbuf[32 * half + 16 * mt + li][32 * kk + 8 * g]));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) {
          // channels 128*w4 + 16*nt + (0..15); rows 32kk + 4g..+3 and 32kk + 16 + 4g..+3
          const int ko = 32 * kk * kPitch + 32 * nt;
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tl3 + t_off0 + ko));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tl3 + t_off1 + ko));
          const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[kk][mt], bv, oacc[mt][nt], 0, 0, 0);
        }
      }
      buf ^= 1;
    }
    if (!overflow) break;
  }

  // ---- finish: publish (m, l) per head
  if (g == 0) {
    sm.lpart[mr][my_head] = l_part;
    if (mr == 0) sm.mfin[my_head] = m_use;
  }
  lds_barrier();
  if (a.splits > 1) {
    // The split's output divided by its own sum (a convex combination of rows, so within
    // the rows' range) goes out as bf16, staged in LDS for 16-byte stores, one 32-head unit
    // per half; attn_combine weighs the splits by their sums.
    uint16_t* ps = reinterpret_cast<uint16_t*>(sm.tile[0]);  // [64][512], contiguous
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float inv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hl = 32 * half + 16 * mt + 4 * g + j;
        const float l = sm.lpart[0][hl] + sm.lpart[1][hl];
        inv[j] = l > 0.f ? 1.0f / l : 0.f;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ps[(32 * half + 16 * mt + 4 * g + j) * kC + 128 * w4 + 16 * nt + li] = f32_to_bf16_bits(oacc[mt][nt][j] * inv[j]);
    }
    auto pidx_of = [&](int h) { return ((size_t)row * a.n_hg + 2 * hg + h) * a.splits + split; };
    if (threadIdx.x < kHW) {
      const int h = threadIdx.x / kHG, hl = threadIdx.x % kHG;
      float* pml = a.part_ml + pidx_of(h) * 2 * kHG;
      pml[hl] = sm.mfin[threadIdx.x];
      pml[kHG + hl] = sm.lpart[0][threadIdx.x] + sm.lpart[1][threadIdx.x];
    }
    lds_barrier();
    const uint4* pl = reinterpret_cast<const uint4*>(ps);
    constexpr int kPerHalf = kHG * kC / 8;
    for (int q = threadIdx.x; q < 2 * kPerHalf; q += kThreadsM) {
      const int h = q / kPerHalf;
      reinterpret_cast<uint4*>(a.part_o + pidx_of(h) * kHG * kC)[q - h * kPerHalf] = pl[q];
    }
    return;
  }
  // single split: normalise, inverse-rotate, stage bf16 output in LDS, coalesced store
  uint16_t* os = reinterpret_cast<uint16_t*>(sm.tile[0]);  // [64][512], contiguous
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    float inv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hl = 32 * half + 16 * mt + 4 * g + j;
      const float l = sm.lpart[0][hl] + sm.lpart[1][hl], m = sm.mfin[hl];
      float den = l;
      if (a.sink && l > 0.f) den += exp2f(a.sink[head0 + hl] * kLog2e - m);
      inv[j] = l > 0.f ? fast_rcp(den) : 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch = 128 * w4 + 16 * nt + li;
      float cs = 1.f, sn = 0.f;
      const bool rot = a.rope_dims > 0 && ch >= rope_lo;
      if (rot) { cs = sm.rope_c[(ch - rope_lo) >> 1]; sn = -sm.rope_s[(ch - rope_lo) >> 1]; }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = oacc[mt][nt][j] * inv[j];
        const float other = dpp<kDppXor1>(v);
        float o = v;
        if (rot) o = (ch & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
        os[(32 * half + 16 * mt + 4 * g + j) * kC + ch] = f32_to_bf16_bits(o);
      }
    }
  }
  if (a.out_mass && threadIdx.x < kHW) {
    const float l = sm.lpart[0][threadIdx.x] + sm.lpart[1][threadIdx.x], m = sm.mfin[threadIdx.x];
    float den = l;
    if (a.sink && l > 0.f) den += exp2f(a.sink[head0 + threadIdx.x] * kLog2e - m);
    a.out_mass[(size_t)row * a.H + head0 + threadIdx.x] = l > 0.f ? l / den : 0.f;
  }
  lds_barrier();
  uint4* op = reinterpret_cast<uint4*>((uint16_t*)a.out + ((size_t)row * a.H + head0) * kC);
  const uint4* src = reinterpret_cast<const uint4*>(os);
  for (int q = threadIdx.x; q < kHW * kC / 8; q += kThreadsM) op[q] = src[q];
}

// merge the splits of one query for 4 heads (one head per wave, 8 channels per lane), in
// split order
constexpr int kCombHeads = 4;
__global__ void __launch_bounds__(256) attn_combine(AttnDev a) {
  __shared__ float rc[64], rs[64];
  const int row = blockIdx.x;
  const int hg = blockIdx.y / (kHG / kCombHeads);
  const int hl = (blockIdx.y % (kHG / kCombHeads)) * kCombHeads + threadIdx.x / 64;
  const int c8 = (threadIdx.x % 64) * 8;
  const int t_pos = a.q_pos[row];
  const int rope_lo = kC - a.rope_dims;
  stage_rope(a, t_pos, rc, rs);
  const size_t pbase = ((size_t)row * a.n_hg + hg) * a.splits;
  const int head0 = hg * kHG;
  // every split's (m, l) and 8 channels are loaded before any is used
  constexpr int kMaxS = 8;
  float ms[kMaxS], ls[kMaxS];
  uint4 xr[kMaxS];
  float mx = -INFINITY, l = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s0 = 0; s0 < a.splits; s0 += kMaxS) {
#pragma unroll
    for (int q = 0; q < kMaxS; ++q) {
      const int s2 = s0 + q;
      if (s2 < a.splits) {
        ms[q] = a.part_ml[(pbase + s2) * 2 * kHG + hl];
        ls[q] = a.part_ml[(pbase + s2) * 2 * kHG + kHG + hl];
        xr[q] = *reinterpret_cast<const uint4*>(a.part_o + ((pbase + s2) * kHG + hl) * kC + c8);
      } else {
        ms[q] = -INFINITY;
      }
    }
    float mnew = mx;
#pragma unroll
    for (int q = 0; q < kMaxS; ++q) mnew = fmaxf(mnew, ms[q]);
    if (mnew == -INFINITY) continue;
    // rescale what earlier groups accumulated (splits merged in order)
    const float r = mx == -INFINITY ? 0.f : exp2f(mx - mnew);
    l *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= r;
    mx = mnew;
#pragma unroll
    for (int q = 0; q < kMaxS; ++q) {
      if (ms[q] == -INFINITY) continue;
      // the split's unnormalised output is its sum times its stored (normalised) output
      const float wl = exp2f(ms[q] - mx) * ls[q];
      l += wl;
      float x[8];
      unpack8(xr[q], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += wl * x[e];
    }
  }
  float den = l;
  if (a.sink && l > 0.f) den += exp2f(a.sink[head0 + hl] * kLog2e - mx);
  const float inv = l > 0.f ? 1.0f / den : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= inv;
  __syncthreads();
  if (a.rope_dims > 0 && c8 + 8 > rope_lo) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int ch = c8 + e;
      if (ch >= rope_lo) {
        const float cs = rc[(ch - rope_lo) >> 1], sn = -rs[(ch - rope_lo) >> 1];
        const float y0 = o[e], y1 = o[e + 1];
        o[e] = y0 * cs - y1 * sn;
        o[e + 1] = y0 * sn + y1 * cs;
      }
    }
  }
  *reinterpret_cast<uint4*>((uint16_t*)a.out + ((size_t)row * a.H + head0 + hl) * kC + c8) = pack8(o);
  if (a.out_mass && c8 == 0) a.out_mass[(size_t)row * a.H + head0 + hl] = l > 0.f ? l * inv : 0.f;
}

bool mfma_ok(const csa2_attn_desc& d) {
  return d.q_dtype == CSA2_BF16 && d.c == kC && d.H % kHW == 0 &&
         (d.kv_dtype == CSA2_BF16 || d.kv_dtype == CSA2_FP4_E4M3) && d.rope_dims <= 128;
}

int max_rows(const csa2_attn_desc& d) { return d.k + ((d.win && d.n_win > 0) ? d.n_win : 0); }

int tile_rows(const csa2_attn_desc& d) { return d.kv_dtype == CSA2_FP4_E4M3 ? kTileOf<true> : kTileOf<false>; }

void pick_splits(const csa2_attn_desc& d, int* splits, int* tps) {
  const int rows = d.B * d.T;
  const int kTile = tile_rows(d);
  const int kMaxSplitTiles = kMaxSplitRows / kTile;
  const int n_tiles = (max_rows(d) + kTile - 1) / kTile;
  const int n_wg = d.H / kHW;  // workgroups per (query, split)
  const int wgs = rows * n_wg;   // 0 for an empty call, which launches nothing
  int s = d.num_splits > 0 ? d.num_splits : (wgs > 0 ? (256 + wgs - 1) / wgs : 1);
  if (s < 1) s = 1;
  if (s > n_tiles) s = n_tiles;
  const int min_s = (n_tiles + kMaxSplitTiles - 1) / kMaxSplitTiles;
  if (s < min_s) s = min_s;
  const int per = (n_tiles + s - 1) / s;
  *tps = per < 1 ? 1 : per;
  *splits = (n_tiles + *tps - 1) / *tps;
  if (*splits < 1) *splits = 1;
}

// dense mode reads every entry slot: N index slots, no index list
csa2_attn_desc effective(const csa2_attn_desc& d0) {
  csa2_attn_desc d = d0;
  if (d.dense_m > 0) d.k = d.N;
  return d;
}

AttnDev make_dev(const csa2_attn_desc& d) {
  AttnDev a{};
  a.B = d.B; a.T = d.T; a.H = d.H; a.c = d.c; a.k = d.k; a.N = d.N; a.rope_dims = d.rope_dims;
  a.q_norm = d.q_norm; a.Lw = d.Lw; a.n_win = d.win ? d.n_win : 0; a.rope_theta = d.rope_theta;
  a.eps = d.eps;
  const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)d.c);
  a.scale_log2 = scale * kLog2e;
  a.q_f32 = d.q_dtype == CSA2_F32;
  a.kv_kind = d.kv_dtype == CSA2_FP4_E4M3 ? 1 : 0;
  a.q = d.q; a.q_pos = d.q_pos; a.kv = d.kv; a.kv_codes = d.kv_codes; a.kv_scales = d.kv_scales;
  a.idx = d.idx; a.win = d.win; a.win_pos0 = d.win_pos0; a.win_row0 = d.win_row0; a.sink = d.sink; a.out = d.out;
  a.out_mass = d.out_mass;
  a.dense_m = d.dense_m;
  a.n_hg = d.H / kHG;
  rope_freq_host(&a.rope, d.rope_dims, d.rope_theta);
  return a;
}


struct AttnPlan {
  int splits, tps;
};
AttnPlan plan_attn(const csa2_attn_desc& d) {
  AttnPlan p{1, 1};
  if (mfma_ok(d)) pick_splits(d, &p.splits, &p.tps);
  return p;
}

}  // namespace

size_t attn_workspace_bytes(const csa2_attn_desc& d0) {
  if ((long long)d0.B * d0.T * d0.H == 0) return 0;
  const csa2_attn_desc d = effective(d0);
  const AttnPlan p = plan_attn(d);
  if (!mfma_ok(d) || p.splits <= 1) return 0;
  const size_t units = (size_t)d.B * d.T * (d.H / kHG);
  return units * p.splits * (kHG * kC * sizeof(uint16_t) + 2 * kHG * sizeof(float));
}

hipError_t launch_attn(const csa2_attn_desc& d0, void* ws, size_t ws_bytes, hipStream_t s) {
  const csa2_attn_desc d = effective(d0);
  const int rows = d.B * d.T;
  if (rows == 0 || d.H == 0) return hipSuccess;
  // every pointer a kernel dereferences must be set
  const bool rows_needed = d.k > 0 && d.N > 0;
  if (!d.q || !d.q_pos || !d.out || (d.k > 0 && !d.idx && d.dense_m == 0) ||
      (rows_needed && d.kv_dtype == CSA2_FP4_E4M3 && (!d.kv_codes || !d.kv_scales)) ||
      (rows_needed && d.kv_dtype != CSA2_FP4_E4M3 && !d.kv) || (d.win && !d.win_pos0 && !d.win_row0))
    return hipErrorInvalidValue;
  AttnDev a = make_dev(d);
  if (!mfma_ok(d)) {
    ScopedProf p(s, "attn_simple");
    if (d.q_dtype == CSA2_F32)
      hipLaunchKernelGGL(attn_simple<float>, dim3(rows * d.H), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(attn_simple<uint16_t>, dim3(rows * d.H), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  const AttnPlan plan = plan_attn(d);
  a.splits = plan.splits;
  a.tiles_per_split = plan.tps;
  if (plan.splits > 1) {
    if (!ws || ws_bytes < attn_workspace_bytes(d)) return hipErrorInvalidValue;
    const size_t units = (size_t)rows * a.n_hg;
    a.part_o = (uint16_t*)ws;
    a.part_ml = (float*)((char*)ws + units * plan.splits * kHG * kC * sizeof(uint16_t));
  }
  const size_t lds_bf16 = sizeof(MfmaSmem<kTileOf<false>>), lds_fp4 = sizeof(MfmaSmem<kTileOf<true>>);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_mfma<false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bf16);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)attn_mfma<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_fp4);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int splits = plan.splits;
  if (d.kv_dtype == CSA2_FP4_E4M3) {
    ScopedProf p(s, "attn_mfma_fp4");
    hipLaunchKernelGGL(attn_mfma<true>, dim3(rows, splits, d.H / kHW), dim3(kThreadsM), lds_fp4, s, a);
  } else {
    ScopedProf p(s, "attn_mfma");
    hipLaunchKernelGGL(attn_mfma<false>, dim3(rows, splits, d.H / kHW), dim3(kThreadsM), lds_bf16, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits <= 1) return e;
  ScopedProf p(s, "attn_combine");
  hipLaunchKernelGGL(attn_combine, dim3(rows, a.n_hg * (kHG / kCombHeads)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2

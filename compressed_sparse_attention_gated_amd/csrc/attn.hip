// Sparse shared-KV MQA over the selected entries plus the sliding window
// ([DSA-to-CSA notes] eq. (18)-(19) and "Shared-KV MQA": every selected entry is both key
// and value, the query heads are RMS-normalised and rotated on the last r dims, the output's
// last r dims are rotated back by the query position; eq. (27): one value-less sink logit
// per head in the softmax denominator; [CSA2 column] "保留了 CSA 的骨架": the selected
// entries are joined by the latest 128 uncompressed rows of the layer).
//
// attn_mfma (bf16 queries, 64-head groups, c = 512, bf16 or FP4 rows):
//   One workgroup = one query x 64 heads x a contiguous range of row slots (a split).
//   Rows are gathered 32 at a time into LDS (FP4 rows dequantised on the way: E2M1 x E4M3
//   is exact in bf16), double-buffered through registers.  Each of the 4 waves owns 16
//   heads for S^T = rows x heads on v_mfma_f32_16x16x32_bf16 (q_hat in registers); the C
//   layout of S^T gives each lane one head and 8 rows, which is exactly the A-operand
//   layout of P for the PV product, so P never needs a transpose.  For PV each wave owns
//   128 output channels of all 64 heads; the V operand (rows along K) is read with the
//   gfx950 LDS transpose read ds_read_b64_tr_b16 from the same row-major tile that fed
//   S^T (shared K = V, one copy in LDS).  Softmax is online in fp32 (exp2, scale folded
//   into q_hat).  Tiles are XOR-swizzled in 16-byte chunks so both read patterns are free
//   of bank conflicts.  With several splits per query the unnormalised partial output and
//   (max, sum) go to a workspace and attn_combine merges them in a fixed order.
//
// attn_simple: any head count / width / dtype; one wave per (query, head), fp32 math.

#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

// ------------------------------------------------------------------ shared row bookkeeping
struct AttnDev {
  int B, T, H, c, k, N, rope_dims, q_norm, Lw, n_win, splits, tiles_per_split, n_hg;
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
  const float* sink;
  void* out;
  float* out_mass;
  float* part_o;   // [rows][n_hg][splits][64][c]
  float* part_ml;  // [rows][n_hg][splits][2][64]
};

struct WinRange {
  int lo_row, cnt;
};
__device__ __forceinline__ WinRange window_of(const AttnDev& a, int b, int t_pos) {
  WinRange w{0, 0};
  if (!a.win || a.n_win <= 0) return w;
  const int p0 = a.win_pos0[b];
  const int lo = max(t_pos - a.n_win + 1, p0);
  const int hi = min(t_pos, p0 + a.Lw - 1);
  if (hi >= lo) { w.lo_row = lo - p0; w.cnt = hi - lo + 1; }
  return w;
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
    const float other = __shfl_xor(qv[j], 1, 64);
    if (a.rope_dims > 0 && ch < c && ch >= c - a.rope_dims) {
      float cs, sn;
      rope_cos_sin((double)t_pos, (ch - (c - a.rope_dims)) / 2, a.rope_dims, a.rope_theta, &cs, &sn);
      qv[j] = (ch & 1) ? (other * sn + qv[j] * cs) : (qv[j] * cs - other * sn);
    }
  }
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) qv[j] *= a.scale_log2;

  const WinRange wr = window_of(a, b, t_pos);
  const int R = a.k + wr.cnt;
  float m_run = -INFINITY, l_run = 0.f;
  float o[kSimpleMaxPerLane];
#pragma unroll
  for (int j = 0; j < kSimpleMaxPerLane; ++j) o[j] = 0.f;
  for (int s = 0; s < R; ++s) {
    float rv[kSimpleMaxPerLane];
    bool valid = true;
    if (s < a.k) {
      const int e = a.idx[(size_t)row * a.k + s];
      valid = e >= 0 && e < a.N;
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
    const float other = __shfl_xor(o[j], 1, 64);
    if (a.rope_dims > 0 && ch < c && ch >= c - a.rope_dims) {
      float cs, sn;
      rope_cos_sin(-(double)t_pos, (ch - (c - a.rope_dims)) / 2, a.rope_dims, a.rope_theta, &cs, &sn);
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
constexpr int kHG = 64;           // heads per workgroup
constexpr int kTile = 32;         // rows per tile
constexpr int kRowBytes = kC * 2;
constexpr int kThreadsM = 256;
constexpr int kChunksPerRow = kRowBytes / 16;  // 64

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// XOR swizzle of the 16-byte chunk index within a row (low 4 bits only)
__device__ __forceinline__ int swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }
__device__ __forceinline__ int chunk_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

struct MfmaSmem {
  // two row tiles; the first 64 KiB also stage q_hat ([64 heads][512] bf16) and, at the
  // end, the bf16 output tile
  alignas(16) uint8_t tile[2][kTile * kRowBytes];
  alignas(16) uint16_t pbuf[kHG][kTile];  // P in PV A-operand order (bf16)
  float alpha[kHG];
  float mfin[kHG], lfin[kHG];
  uint32_t vmask[2];
  int src_row[2][kTile];  // per tile row: >= 0 kv entry id, -2-w window row w, -1 empty
};

// fetch registers for one tile: each thread holds up to 8 chunks (bf16 rows) or 2 FP4
// code chunks + their 2 scale bytes
struct Prefetch {
  uint4 v[8];
  uint4 fc[2];
  uint32_t fs[2];
};

__device__ __forceinline__ void resolve_rows(const AttnDev& a, int row, int b, int slot0, int slot_end,
                                             const WinRange& wr, int* src) {
  // one thread per tile row
  const int r = threadIdx.x;
  if (r < kTile) {
    const int s = slot0 + r;
    int v = -1;
    if (s < slot_end) {
      if (s < a.k) {
        const int e = a.idx[(size_t)row * a.k + s];
        v = (e >= 0 && e < a.N) ? e : -1;
      } else {
        v = -2 - (wr.lo_row + (s - a.k));
      }
    }
    src[r] = v;
  }
}

__device__ __forceinline__ void fetch_tile(const AttnDev& a, int b, const int* src, Prefetch& pf) {
  const int tid = threadIdx.x;
  // bf16 rows (kv rows when bf16, window rows always): chunk q = tid + 256*i -> row q/64
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 6) + 4 * i, ch = tid & 63;
    const int sr = src[r];
    const uint16_t* base = nullptr;
    if (sr <= -2) base = (const uint16_t*)a.win + ((size_t)b * a.Lw + (-2 - sr)) * kC;
    else if (sr >= 0 && a.kv_kind == 0) base = (const uint16_t*)a.kv + ((size_t)b * a.N + sr) * kC;
    pf.v[i] = base ? reinterpret_cast<const uint4*>(base)[ch] : make_uint4(0, 0, 0, 0);
  }
  if (a.kv_kind == 1) {
    // FP4 rows: 16 code chunks of 16 B per row -> q = tid + 256*i, row q/16, part q%16
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      const int r = q >> 4, part = q & 15;
      const int sr = src[r];
      if (sr >= 0) {
        pf.fc[i] = reinterpret_cast<const uint4*>(a.kv_codes + ((size_t)b * a.N + sr) * (kC / 2))[part];
        const uint8_t* sp = a.kv_scales + ((size_t)b * a.N + sr) * (kC / 16) + 2 * part;
        pf.fs[i] = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
      } else {
        pf.fc[i] = make_uint4(0, 0, 0, 0);
        pf.fs[i] = 0;
      }
    }
  }
}

__device__ __forceinline__ void commit_tile(const AttnDev& a, const int* src, const Prefetch& pf, uint8_t* tile) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 6) + 4 * i, ch = tid & 63;
    const int sr = src[r];
    if (sr <= -2 || sr == -1 || a.kv_kind == 0)
      *reinterpret_cast<uint4*>(tile + chunk_off(r, ch)) = pf.v[i];
  }
  if (a.kv_kind == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      const int r = q >> 4, part = q & 15;
      if (src[r] >= 0) {
        // 32 codes -> channels 32*part .. 32*part+31, scales for groups 2*part, 2*part+1
        const float s0 = e4m3_to_f32(pf.fs[i] & 0xffu), s1 = e4m3_to_f32(pf.fs[i] >> 8);
        const uint32_t words[4] = {pf.fc[i].x, pf.fc[i].y, pf.fc[i].z, pf.fc[i].w};
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          float f[8];
          const float sc = qq < 2 ? s0 : s1;
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = e2m1_to_f32((words[qq] >> (4 * e)) & 15u) * sc;
          *reinterpret_cast<uint4*>(tile + chunk_off(r, 4 * part + qq)) = pack8(f);
        }
      }
    }
  }
}

__global__ void __launch_bounds__(kThreadsM) attn_mfma(AttnDev a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  MfmaSmem& sm = *reinterpret_cast<MfmaSmem*>(smem_raw);
  const int split = blockIdx.y;
  const int hg = blockIdx.z;
  const int row = blockIdx.x;
  const int b = row / a.T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int t_pos = a.q_pos[row];
  const WinRange wr = window_of(a, b, t_pos);
  const int R = a.k + wr.cnt;
  const int n_tiles = (R + kTile - 1) / kTile;
  const int tile0 = split * a.tiles_per_split;
  const int tile1 = min(tile0 + a.tiles_per_split, n_tiles);

  // ---- q_hat for this wave's 16 heads -> LDS (bf16) -> B-operand registers
  uint16_t* qs = reinterpret_cast<uint16_t*>(sm.tile[0]);  // [64][512]
  for (int hh = 0; hh < 16; ++hh) {
    const int hl = 16 * wave + hh;
    const int head = hg * kHG + hl;
    const uint16_t* qp = (const uint16_t*)a.q + ((size_t)row * a.H + head) * kC + 8 * lane;
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(qp), f);
    if (a.q_norm) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)kC + a.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= inv;
    }
    if (a.rope_dims > 0 && 8 * lane + 8 > kC - a.rope_dims) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int ch = 8 * lane + e;
        if (ch >= kC - a.rope_dims) {
          float cs, sn;
          rope_cos_sin((double)t_pos, (ch - (kC - a.rope_dims)) / 2, a.rope_dims, a.rope_theta, &cs, &sn);
          const float x0 = f[e], x1 = f[e + 1];
          f[e] = x0 * cs - x1 * sn;
          f[e + 1] = x0 * sn + x1 * cs;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] *= a.scale_log2;
    *reinterpret_cast<uint4*>(qs + hl * kC + 8 * lane) = pack8(f);
  }
  __syncthreads();
  bf16x8 qreg[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
    qreg[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qs + (16 * wave + li) * kC + 32 * ks + 8 * g));
  __syncthreads();

  // ---- state
  float m_run = -INFINITY, l_run = 0.f;  // head 16*wave + li (replicated over g)
  f32x4 oacc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  Prefetch pf;
  if (tile0 < tile1) {
    resolve_rows(a, row, b, tile0 * kTile, R, wr, sm.src_row[0]);
    __syncthreads();
    fetch_tile(a, b, sm.src_row[0], pf);
  }
  int buf = 0;
  for (int ti = tile0; ti < tile1; ++ti) {
    commit_tile(a, sm.src_row[buf], pf, sm.tile[buf]);
    if (threadIdx.x == 0) {
      uint32_t vm = 0;
      for (int r = 0; r < kTile; ++r) vm |= (sm.src_row[buf][r] != -1 ? 1u : 0u) << r;
      sm.vmask[buf] = vm;
    }
    const bool more = ti + 1 < tile1;
    if (more) resolve_rows(a, row, b, (ti + 1) * kTile, R, wr, sm.src_row[buf ^ 1]);
    __syncthreads();
    if (more) fetch_tile(a, b, sm.src_row[buf ^ 1], pf);

    const uint8_t* tl = sm.tile[buf];
    const lds_u8* tl3 = (const lds_u8*)tl;  // LDS view for the transpose reads
    const uint32_t vm = sm.vmask[buf];
    // ---- S^T = rows x heads for this wave's 16 heads (two 16-row M tiles)
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int mr = 0; mr < 2; ++mr) {
      const int r = 16 * mr + li;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4*>(tl + chunk_off(r, 4 * ks + g)));
        sacc[mr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[ks], sacc[mr], 0, 0, 0);
      }
    }
    // lane holds head 16*wave+li, rows 16*mr + 4*g + j
    float tmax = -INFINITY;
#pragma unroll
    for (int mr = 0; mr < 2; ++mr)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((vm >> (16 * mr + 4 * g + j)) & 1u) tmax = fmaxf(tmax, sacc[mr][j]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == m_run) ? 1.0f : exp2f(m_run - m_new);
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int mr = 0; mr < 2; ++mr)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool v = (vm >> (16 * mr + 4 * g + j)) & 1u;
        const float pv = v ? exp2f(sacc[mr][j] - m_new) : 0.f;
        p[4 * mr + j] = pv;
        psum += pv;
      }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // P for head 16*wave+li, k-slots 8g..8g+7 = rows {4g..4g+3, 16+4g..16+4g+3}
    *reinterpret_cast<uint4*>(&sm.pbuf[16 * wave + li][8 * g]) = pack8(p);
    if (g == 0) sm.alpha[16 * wave + li] = alpha;
    __syncthreads();

    // ---- O[:, 128*wave .. +128] = O * alpha + P x V
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float al[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) al[j] = sm.alpha[16 * mt + 4 * g + j];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) oacc[mt][nt][j] *= al[j];
    }
    bf16x8 pa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) pa[mt] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.pbuf[16 * mt + li][8 * g]));
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch_base = 128 * wave + 16 * nt;
      // source lane (g, s=li): row base + li/4, channels ch_base + 4*(li%4) .. +3
      const int chunk = (ch_base >> 3) + ((li & 3) >> 1);
      const int within = 8 * (li & 1);
      const int r0 = 4 * g + (li >> 2);
      const int r1 = 16 + 4 * g + (li >> 2);
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tl3 + chunk_off(r0, chunk) + within));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tl3 + chunk_off(r1, chunk) + within));
      const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        oacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mt], bv, oacc[mt][nt], 0, 0, 0);
    }
    buf ^= 1;
  }

  // ---- finish: publish (m, l) per head
  if (g == 0) { sm.mfin[16 * wave + li] = m_run; sm.lfin[16 * wave + li] = l_run; }
  __syncthreads();
  const int head0 = hg * kHG;
  if (a.splits > 1) {
    const size_t pidx = ((size_t)row * a.n_hg + hg) * a.splits + split;
    float* po = a.part_o + pidx * kHG * kC;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          po[(size_t)(16 * mt + 4 * g + j) * kC + 128 * wave + 16 * nt + li] = oacc[mt][nt][j];
    if (threadIdx.x < kHG) {
      float* pml = a.part_ml + pidx * 2 * kHG;
      pml[threadIdx.x] = sm.mfin[threadIdx.x];
      pml[kHG + threadIdx.x] = sm.lfin[threadIdx.x];
    }
    return;
  }
  // single split: normalise, inverse-rotate, stage bf16 output in LDS, coalesced store
  uint16_t* os = reinterpret_cast<uint16_t*>(sm.tile[0]);  // [64][512]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    float inv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hl = 16 * mt + 4 * g + j;
      const float l = sm.lfin[hl], m = sm.mfin[hl];
      float den = l;
      if (a.sink && l > 0.f) den += exp2f(a.sink[head0 + hl] * kLog2e - m);
      inv[j] = l > 0.f ? 1.0f / den : 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch = 128 * wave + 16 * nt + li;
      float cs = 1.f, sn = 0.f;
      const bool rot = a.rope_dims > 0 && ch >= kC - a.rope_dims;
      if (rot) rope_cos_sin(-(double)t_pos, (ch - (kC - a.rope_dims)) / 2, a.rope_dims, a.rope_theta, &cs, &sn);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = oacc[mt][nt][j] * inv[j];
        const float other = __shfl_xor(v, 1, 64);
        float o = v;
        if (rot) o = (ch & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
        os[(16 * mt + 4 * g + j) * kC + ch] = f32_to_bf16_bits(o);
      }
    }
  }
  if (a.out_mass && threadIdx.x < kHG) {
    const float l = sm.lfin[threadIdx.x], m = sm.mfin[threadIdx.x];
    float den = l;
    if (a.sink && l > 0.f) den += exp2f(a.sink[head0 + threadIdx.x] * kLog2e - m);
    a.out_mass[(size_t)row * a.H + head0 + threadIdx.x] = l > 0.f ? l / den : 0.f;
  }
  __syncthreads();
  uint4* op = reinterpret_cast<uint4*>((uint16_t*)a.out + ((size_t)row * a.H + head0) * kC);
  const uint4* src = reinterpret_cast<const uint4*>(os);
  for (int q = threadIdx.x; q < kHG * kC / 8; q += kThreadsM) op[q] = src[q];
}

// merge the splits of one (query, 64-head group) in split order
__global__ void __launch_bounds__(256) attn_combine(AttnDev a) {
  const int row = blockIdx.x, hg = blockIdx.y;
  const int t_pos = a.q_pos[row];
  const size_t pbase = ((size_t)row * a.n_hg + hg) * a.splits;
  const int head0 = hg * kHG;
  for (int q = threadIdx.x; q < kHG * kC / 8; q += 256) {
    const int hl = q / (kC / 8), c8 = (q % (kC / 8)) * 8;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.part_ml[(pbase + s) * 2 * kHG + hl]);
    float l = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (mx != -INFINITY) {
      for (int s = 0; s < a.splits; ++s) {
        const float ms = a.part_ml[(pbase + s) * 2 * kHG + hl];
        if (ms == -INFINITY) continue;
        const float wgt = exp2f(ms - mx);
        l += wgt * a.part_ml[(pbase + s) * 2 * kHG + kHG + hl];
        const float4* po = reinterpret_cast<const float4*>(a.part_o + ((pbase + s) * kHG + hl) * kC + c8);
        const float4 x0 = po[0], x1 = po[1];
        o[0] += wgt * x0.x; o[1] += wgt * x0.y; o[2] += wgt * x0.z; o[3] += wgt * x0.w;
        o[4] += wgt * x1.x; o[5] += wgt * x1.y; o[6] += wgt * x1.z; o[7] += wgt * x1.w;
      }
    }
    float den = l;
    if (a.sink && l > 0.f) den += exp2f(a.sink[head0 + hl] * kLog2e - mx);
    const float inv = l > 0.f ? 1.0f / den : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
    if (a.rope_dims > 0 && c8 + 8 > kC - a.rope_dims) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int ch = c8 + e;
        if (ch >= kC - a.rope_dims) {
          float cs, sn;
          rope_cos_sin(-(double)t_pos, (ch - (kC - a.rope_dims)) / 2, a.rope_dims, a.rope_theta, &cs, &sn);
          const float x0 = o[e], x1 = o[e + 1];
          o[e] = x0 * cs - x1 * sn;
          o[e + 1] = x0 * sn + x1 * cs;
        }
      }
    }
    *reinterpret_cast<uint4*>((uint16_t*)a.out + ((size_t)row * a.H + head0 + hl) * kC + c8) = pack8(o);
    if (a.out_mass && c8 == 0) a.out_mass[(size_t)row * a.H + head0 + hl] = l > 0.f ? l * inv : 0.f;
  }
}

bool mfma_ok(const csa2_attn_desc& d) {
  return d.q_dtype == CSA2_BF16 && d.c == kC && d.H % kHG == 0 &&
         (d.kv_dtype == CSA2_BF16 || d.kv_dtype == CSA2_FP4_E4M3) && d.rope_dims <= 128;
}

int max_rows(const csa2_attn_desc& d) { return d.k + ((d.win && d.n_win > 0) ? d.n_win : 0); }

void pick_splits(const csa2_attn_desc& d, int* splits, int* tps) {
  const int rows = d.B * d.T;
  const int n_tiles = (max_rows(d) + kTile - 1) / kTile;
  const int n_hg = d.H / kHG;
  int s = d.num_splits > 0 ? d.num_splits : (512 + rows * n_hg - 1) / (rows * n_hg);
  if (s < 1) s = 1;
  if (s > n_tiles) s = n_tiles;
  const int per = (n_tiles + s - 1) / s;
  *tps = per < 1 ? 1 : per;
  *splits = (n_tiles + *tps - 1) / *tps;
  if (*splits < 1) *splits = 1;
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
  a.idx = d.idx; a.win = d.win; a.win_pos0 = d.win_pos0; a.sink = d.sink; a.out = d.out;
  a.out_mass = d.out_mass;
  a.n_hg = d.H / kHG;
  return a;
}

}  // namespace

size_t attn_workspace_bytes(const csa2_attn_desc& d) {
  if (!mfma_ok(d)) return 0;
  int splits, tps;
  pick_splits(d, &splits, &tps);
  if (splits <= 1) return 0;
  const size_t units = (size_t)d.B * d.T * (d.H / kHG) * splits;
  return units * (kHG * kC + 2 * kHG) * sizeof(float);
}

hipError_t launch_attn(const csa2_attn_desc& d, void* ws, size_t ws_bytes, hipStream_t s) {
  const int rows = d.B * d.T;
  if (rows == 0 || d.H == 0) return hipSuccess;
  // every pointer a kernel dereferences must be set
  const bool rows_needed = d.k > 0 && d.N > 0;
  if (!d.q || !d.q_pos || !d.out || (d.k > 0 && !d.idx) ||
      (rows_needed && d.kv_dtype == CSA2_FP4_E4M3 && (!d.kv_codes || !d.kv_scales)) ||
      (rows_needed && d.kv_dtype != CSA2_FP4_E4M3 && !d.kv) || (d.win && !d.win_pos0))
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
  int splits, tps;
  pick_splits(d, &splits, &tps);
  a.splits = splits;
  a.tiles_per_split = tps;
  if (splits > 1) {
    if (!ws || ws_bytes < attn_workspace_bytes(d)) return hipErrorInvalidValue;
    const size_t units = (size_t)rows * a.n_hg * splits;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + units * kHG * kC * sizeof(float));
    (void)ws_bytes;
  }
  const size_t lds = sizeof(MfmaSmem);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_mfma, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  {
    ScopedProf p(s, d.kv_dtype == CSA2_FP4_E4M3 ? "attn_mfma_fp4" : "attn_mfma");
    hipLaunchKernelGGL(attn_mfma, dim3(rows, splits, a.n_hg), dim3(kThreadsM), lds, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits <= 1) return e;
  ScopedProf p(s, "attn_combine");
  hipLaunchKernelGGL(attn_combine, dim3(rows, a.n_hg), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2

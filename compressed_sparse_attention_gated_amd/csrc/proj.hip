// Grouped output projection after the core attention ([DSA-to-CSA notes], section "Grouped
// output projection"): the n_h heads' outputs are split into g groups of n_h/g consecutive
// heads; group j's c*n_h/g values are projected to d_g, and the g*d_g concatenation is
// projected to d.  Both levels are C = A * W^T products with the weights stored (output,
// input), so each operand row is contiguous along the contraction and feeds the MFMA
// operands straight from memory:
//   level 1: g products in one launch (blockIdx.z = group), A = the group's slice of the
//            attention output rows, C = the group's slice of `mid`;
//   level 2: one product, A = mid.
//
// gemm_nt: a wave owns a 32 x 64 tile of C as two v_mfma_f32_32x32x16_bf16 accumulators.
// Lane l reads row l % 32 of A and of each 32-row W block, 16 bytes at k offset 8 * (l / 32)
// of every 16-wide k step (the MFMA operand layout), through a 4-deep ring of 32-k steps.
// Rows past M or N are read clamped and never stored.  Workgroup = 4 waves, 2 x 2 (1 x 4
// along N when M <= 32).  It serves the shapes the two kernels below do not: few rows with a
// contraction that does not split evenly (gemm_nt_splitk), many rows (gemm_nt_lds).

#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kPT = 256;
constexpr int kKStep = 32;  // k per pipeline step (2 MFMA steps of 16)
constexpr int kDepth = 4;   // pipeline steps in flight

struct GemmArgs {
  int M, N, K;
  const uint16_t* A;
  int64_t lda, sa;  // row stride, batch stride (elements)
  const uint16_t* W;
  int64_t sw;       // batch stride; rows are K long
  uint16_t* C;
  int64_t ldc, sc;
};

template <int WM, int WN>
__global__ void __launch_bounds__(kPT) gemm_nt(GemmArgs p) {
  const int z = blockIdx.z;
  const uint16_t* A = p.A + z * p.sa;
  const uint16_t* W = p.W + z * p.sw;
  uint16_t* Cz = p.C + z * p.sc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int m0 = blockIdx.y * 32 * WM + 32 * wm;
  const int n0 = blockIdx.x * 64 * WN + 64 * wn;
  const int r = lane & 31, h = lane >> 5;
  const uint16_t* pa = A + (size_t)min(m0 + r, p.M - 1) * p.lda + 8 * h;
  const uint16_t* pw0 = W + (size_t)min(n0 + r, p.N - 1) * p.K + 8 * h;
  const uint16_t* pw1 = W + (size_t)min(n0 + 32 + r, p.N - 1) * p.K + 8 * h;
  const int nk = p.K / kKStep;
  f32x16 acc0 = {}, acc1 = {};
  // k steps of 32 through a kDepth-deep register ring: step t is used while the next
  // kDepth - 1 load.  Each load goes into the slot just used (no copies for the compiler to
  // fold back into load-then-wait), every trip issues the same loads (steps past the end
  // reload the last one, never used), and the last steps drain after the loop.
  struct Raw {
    uint4 a[2], w0[2], w1[2];
  };
  auto load = [&](int t, Raw& q) {
    const int k = min(t, nk - 1) * kKStep;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      q.a[s] = *reinterpret_cast<const uint4*>(pa + k + 16 * s);
      q.w0[s] = *reinterpret_cast<const uint4*>(pw0 + k + 16 * s);
      q.w1[s] = *reinterpret_cast<const uint4*>(pw1 + k + 16 * s);
    }
  };
  auto use = [&](const Raw& q) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(q.a[s]), as_bf16x8(q.w0[s]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(q.a[s]), as_bf16x8(q.w1[s]), acc1, 0, 0, 0);
    }
  };
  Raw ring[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) {
    load(i, ring[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int t = 0;
  for (; t + kDepth - 1 < nk; t += kDepth) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      load(t + i + kDepth - 1, ring[(i + kDepth - 1) % kDepth]);
      use(ring[i]);
    }
  }
  // ring[i] holds step t + i; fewer than kDepth of them are below nk
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) {
    if (t + i >= nk) break;
    use(ring[i]);
  }
  // C layout of a 32 x 32 accumulator: lane l holds column l % 32, register i row
  // 8 * (i / 4) + 4 * (l / 32) + i % 4
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + 8 * (i / 4) + 4 * h + (i % 4);
    if (m >= p.M) continue;
    uint16_t* crow = Cz + (size_t)m * p.ldc;
    if (n0 + r < p.N) crow[n0 + r] = f32_to_bf16_bits(acc0[i]);
    if (n0 + 32 + r < p.N) crow[n0 + 32 + r] = f32_to_bf16_bits(acc1[i]);
  }
}

// Few rows (decode: one token per sequence): the product is a stream over the weights.  A
// workgroup of kSplit waves owns a 16MB x 16NB tile of C as MB x NB 16 x 16 accumulators
// (MB = 2 for up to 32 rows, 4 for up to 64); wave w takes the w-th 1/kSplit of the
// contraction through the same register ring, and the partial tiles meet in LDS, added in
// wave order (deterministic).  The 16 x 16 x 32 layout gives each load 64 contiguous bytes
// of 16 rows (the 32 x 32 x 16 one gives 32 bytes of 32 rows), which streams the weights
// faster.  NB = 2 when N/32 x batch workgroups still fill the 256 compute units, else NB = 1;
// each workgroup reads its weight rows once.
constexpr int kSplit = 8;
constexpr int kSplitRows = 64;  // most rows the split-K kernel takes
template <int MB, int NB>  // 16-row blocks (2 or 4), 16-column blocks (1 or 2) per workgroup
__global__ void __launch_bounds__(64 * kSplit) gemm_nt_splitk(GemmArgs p) {
  __shared__ float part[kSplit][4 * MB * NB][64];
  const int z = blockIdx.z;
  const uint16_t* A = p.A + z * p.sa;
  const uint16_t* W = p.W + z * p.sw;
  uint16_t* Cz = p.C + z * p.sc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16 * NB;
  // 16 x 16 x 32 operand layout: lane l reads row l % 16 of a 16-row block, the 8 k values
  // at 8 * (l / 16) of every 32-wide k step, so one load covers 64 contiguous bytes of 16 rows
  const int r = lane & 15, c = lane >> 4;
  const int kspan = p.K / kSplit;
  const size_t k0 = (size_t)wave * kspan + 8 * c;
  const uint16_t* pa[MB];
  const uint16_t* pw[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) pa[mb] = A + (size_t)min(16 * mb + r, p.M - 1) * p.lda + k0;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) pw[nb] = W + (size_t)min(n0 + 16 * nb + r, p.N - 1) * p.K + k0;
  const int nk = kspan / kKStep;
  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  struct Raw {
    uint4 a[MB], w[NB];
  };
  auto load = [&](int t, Raw& q) {
    const int k = min(t, nk - 1) * kKStep;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) q.a[mb] = *reinterpret_cast<const uint4*>(pa[mb] + k);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) q.w[nb] = *reinterpret_cast<const uint4*>(pw[nb] + k);
  };
  auto use = [&](const Raw& q) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(q.a[mb]), as_bf16x8(q.w[nb]), acc[mb][nb], 0, 0, 0);
  };
  Raw ring[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) {
    load(i, ring[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int t = 0;
  for (; t + kDepth - 1 < nk; t += kDepth) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      load(t + i + kDepth - 1, ring[(i + kDepth - 1) % kDepth]);
      use(ring[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) {
    if (t + i >= nk) break;
    use(ring[i]);
  }
  // C layout of a 16 x 16 accumulator: lane l holds column l % 16, register i row
  // 4 * (l / 16) + i; partial slot 4 * (NB * row block + column block) + i
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][4 * (NB * mb + nb) + i][lane] = acc[mb][nb][i];
  __syncthreads();
  // thread (j, l) of the first 4MB*NB x 64 adds the waves' slot j of lane l, in wave order
  for (int e = threadIdx.x; e < 4 * MB * NB * 64; e += 64 * kSplit) {
    const int j = e / 64, l = e % 64;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kSplit; ++w) v += part[w][j][l];
    const int mb = j / (4 * NB), nb = (j / 4) % NB, i = j % 4;
    const int m = 16 * mb + 4 * (l / 16) + i, n = n0 + 16 * nb + (l % 16);
    if (m < p.M && n < p.N) Cz[(size_t)m * p.ldc + n] = f32_to_bf16_bits(v);
  }
}

// Many rows (prefill): a 128 x 128 tile of C per workgroup of 4 waves (2 x 2, each 64 x 64
// as 2 x 2 accumulators), the operands shared through LDS.  k stages of 64 are loaded
// coalesced (8 threads per 128-byte row) into registers two stages ahead, then stored into
// the LDS buffer the stage is used from; one barrier per stage.  Rows are padded to 144
// bytes so the 16-byte operand reads of 8 consecutive rows fall in distinct banks.
constexpr int kTM = 128, kTN = 128, kTK = 64;
constexpr int kLdsPitch = kTK + 8;  // bf16 elements per LDS row
__global__ void __launch_bounds__(256, 2) gemm_nt_lds(GemmArgs p) {
  __shared__ __align__(16) uint16_t As[2][kTM][kLdsPitch];
  __shared__ __align__(16) uint16_t Ws[2][kTN][kLdsPitch];
  const int z = blockIdx.z;
  const uint16_t* A = p.A + z * p.sa;
  const uint16_t* W = p.W + z * p.sw;
  uint16_t* Cz = p.C + z * p.sc;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.y * kTM, n0 = blockIdx.x * kTN;
  const int r = lane & 31, h = lane >> 5;
  // global -> register staging: thread covers 16-byte column (tid % 8) of rows tid / 8 + 32 i
  const int gc = tid & 7, gr = tid >> 3;
  const uint16_t* ga[4];
  const uint16_t* gw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ga[i] = A + (size_t)min(m0 + gr + 32 * i, p.M - 1) * p.lda + 8 * gc;
    gw[i] = W + (size_t)min(n0 + gr + 32 * i, p.N - 1) * p.K + 8 * gc;
  }
  const int nkt = p.K / kTK;
  // two register sets of named values (arrays here were placed in scratch memory): stage kt
  // travels in set kt & 1, loaded one full stage before it is stored into LDS
  uint4 a00, a01, a02, a03, w00, w01, w02, w03;  // set 0
  uint4 a10, a11, a12, a13, w10, w11, w12, w13;  // set 1
  f32x16 acc[2][2] = {};
#define CSA2_LD(P, i, k_) (*reinterpret_cast<const uint4*>(P[i] + (k_)))
#define CSA2_GLOAD(S, kt_)                                                               \
  do {                                                                                   \
    const int k_ = min((kt_), nkt - 1) * kTK;                                            \
    a##S##0 = CSA2_LD(ga, 0, k_); a##S##1 = CSA2_LD(ga, 1, k_);                          \
    a##S##2 = CSA2_LD(ga, 2, k_); a##S##3 = CSA2_LD(ga, 3, k_);                          \
    w##S##0 = CSA2_LD(gw, 0, k_); w##S##1 = CSA2_LD(gw, 1, k_);                          \
    w##S##2 = CSA2_LD(gw, 2, k_); w##S##3 = CSA2_LD(gw, 3, k_);                          \
  } while (0)
#define CSA2_ST(buf_, i, A_, W_)                                                         \
  do {                                                                                   \
    *reinterpret_cast<uint4*>(&As[buf_][gr + 32 * (i)][8 * gc]) = A_;                    \
    *reinterpret_cast<uint4*>(&Ws[buf_][gr + 32 * (i)][8 * gc]) = W_;                    \
  } while (0)
#define CSA2_LSTORE(S, buf_)                                                             \
  do {                                                                                   \
    CSA2_ST(buf_, 0, a##S##0, w##S##0); CSA2_ST(buf_, 1, a##S##1, w##S##1);              \
    CSA2_ST(buf_, 2, a##S##2, w##S##2); CSA2_ST(buf_, 3, a##S##3, w##S##3);              \
  } while (0)
#define CSA2_COMPUTE(cur_)                                                                             \
  do {                                                                                                 \
    _Pragma("unroll") for (int s = 0; s < kTK / 16; ++s) {                                             \
      bf16x8 af[2], wf[2];                                                                             \
      _Pragma("unroll") for (int b = 0; b < 2; ++b) {                                                  \
        af[b] = as_bf16x8(*reinterpret_cast<const uint4*>(&As[cur_][64 * wm + 32 * b + r][16 * s + 8 * h])); \
        wf[b] = as_bf16x8(*reinterpret_cast<const uint4*>(&Ws[cur_][64 * wn + 32 * b + r][16 * s + 8 * h])); \
      }                                                                                                \
      _Pragma("unroll") for (int bm = 0; bm < 2; ++bm)                                                 \
      _Pragma("unroll") for (int bn = 0; bn < 2; ++bn)                                                 \
        acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bm], wf[bn], acc[bm][bn], 0, 0, 0);   \
    }                                                                                                  \
  } while (0)
  CSA2_GLOAD(0, 0);
  CSA2_LSTORE(0, 0);
  CSA2_GLOAD(1, 1);
  __syncthreads();
  // loads past the last stage reload it (never stored), so every trip issues the same loads
  for (int kt = 0; kt < nkt; kt += 2) {
    CSA2_GLOAD(0, kt + 2);                      // set 0 was stored last trip
    CSA2_COMPUTE(0);
    if (kt + 1 < nkt) CSA2_LSTORE(1, 1);        // buffer 1: last read before the previous barrier
    __syncthreads();
    if (kt + 1 >= nkt) break;
    CSA2_GLOAD(1, kt + 3);
    CSA2_COMPUTE(1);
    if (kt + 2 < nkt) CSA2_LSTORE(0, 0);
    __syncthreads();
  }
#undef CSA2_LD
#undef CSA2_GLOAD
#undef CSA2_ST
#undef CSA2_LSTORE
#undef CSA2_COMPUTE
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + 64 * wm + 32 * bm + 8 * (i / 4) + 4 * h + (i % 4);
        const int n = n0 + 64 * wn + 32 * bn + r;
        if (m < p.M && n < p.N) Cz[(size_t)m * p.ldc + n] = f32_to_bf16_bits(acc[bm][bn][i]);
      }
}

hipError_t launch_gemm(const GemmArgs& p, int batch, hipStream_t s, const char* name) {
  ScopedProf prof(s, name);
  if (p.M <= kSplitRows && p.K % (kSplit * kKStep) == 0) {
    // 32 columns per workgroup when that still gives one per compute unit, else 16
    const bool wide = (size_t)((p.N + 31) / 32) * batch >= 256;
    const dim3 grid(wide ? (p.N + 31) / 32 : (p.N + 15) / 16, 1, batch), block(64 * kSplit);
    if (p.M <= 32) {
      if (wide) hipLaunchKernelGGL((gemm_nt_splitk<2, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((gemm_nt_splitk<2, 1>), grid, block, 0, s, p);
    } else {
      if (wide) hipLaunchKernelGGL((gemm_nt_splitk<4, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((gemm_nt_splitk<4, 1>), grid, block, 0, s, p);
    }
  } else if (p.M > 32 && p.K % kTK == 0) {
    dim3 grid((p.N + kTN - 1) / kTN, (p.M + kTM - 1) / kTM, batch);
    hipLaunchKernelGGL(gemm_nt_lds, grid, dim3(256), 0, s, p);
  } else if (p.M <= 32) {
    dim3 grid((p.N + 255) / 256, (p.M + 31) / 32, batch);
    hipLaunchKernelGGL((gemm_nt<1, 4>), grid, dim3(kPT), 0, s, p);
  } else {
    dim3 grid((p.N + 127) / 128, (p.M + 63) / 64, batch);
    hipLaunchKernelGGL((gemm_nt<2, 2>), grid, dim3(kPT), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_out_proj(const csa2_out_proj_desc& d, hipStream_t s) {
  if (d.M == 0) return hipSuccess;
  if (!d.o || !d.w1 || !d.w2 || !d.mid || !d.out) return hipErrorInvalidValue;
  const int kg = d.c * (d.n_h / d.g);  // inputs per group
  const int k2 = d.g * d.d_g;
  GemmArgs l1{d.M, d.d_g, kg, (const uint16_t*)d.o, (int64_t)d.n_h * d.c, kg,
              (const uint16_t*)d.w1, (int64_t)d.d_g * kg, (uint16_t*)d.mid, k2, d.d_g};
  hipError_t e = launch_gemm(l1, d.g, s, "out_proj_groups");
  if (e != hipSuccess) return e;
  GemmArgs l2{d.M, d.d, k2, (const uint16_t*)d.mid, k2, 0, (const uint16_t*)d.w2, 0, (uint16_t*)d.out, d.d, 0};
  return launch_gemm(l2, 1, s, "out_proj_concat");
}

}  // namespace csa2

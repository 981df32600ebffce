// GEMMs of the MM-DiT block: C[M, N] = A[M, K] . W[N, K]^T with fused
// epilogues (bias; gated residual h += gate * y; SwiGLU silu(y1) * y3).
//
// These are the per-stream Linear layers of each block (img_qkv / txt_qkv,
// to_out / to_add_out, img_mlp / txt_mlp w1 w3 w2 in the Lens-Turbo-3.8B-bf16
// article; the gated residual and gated MLP of the Lens blog's "Overview").
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation.  A
// 256-thread workgroup (4 waves, 2 x 2) computes a BM x BN tile; each wave
// holds (BM/2) x (BN/2) accumulators.  K advances in steps of 64 through a
// double-buffered LDS tile (rows padded by 16 bytes so the 16-byte fragment
// reads of 32 consecutive rows do not collide in LDS banks).  Both operands
// are K-contiguous, so every global load and every LDS fragment read is a
// 16-byte vector.  Image and text problems (different weights, different M)
// run in one grouped launch.
//
// fp32 path: a plain LDS-tiled FMA kernel with the same epilogues, used by
// the fp32 configuration (correctness, not speed).
#include "common.h"

namespace lens {

namespace {

constexpr int BK = 64;
constexpr int LDS_PAD = 8;            // bf16 elements of padding per LDS row
constexpr int LROW = BK + LDS_PAD;    // LDS row stride in bf16 elements

// Store one output element (non-SwiGLU epilogues).
template <int EPI, typename T>
__device__ __forceinline__ void epi_store(const GemmProblem &p, int m, int n, float acc) {
  float y = acc;
  if (p.bias) y += to_f32(((const T *)p.bias)[n]);
  if constexpr (EPI == EPI_STORE) {
    ((T *)p.C)[(int64_t)m * p.N + n] = from_f32<T>(y);
  } else if constexpr (EPI == EPI_STORE_F32) {
    ((float *)p.C)[(int64_t)m * p.N + n] = y;
  } else if constexpr (EPI == EPI_GATED) {
    const float g = p.gate[(int64_t)(m / p.rows_per_gate) * p.gate_stride + n];
    float *h = (float *)p.C + (int64_t)m * p.N + n;
    *h = *h + g * y;
  }
}

template <typename T>
__device__ __forceinline__ void epi_swiglu(const GemmProblem &p, int m, int n, float a1, float a3) {
  float g = a1, u = a3;
  if (p.bias) g += to_f32(((const T *)p.bias)[n]);
  if (p.bias3) u += to_f32(((const T *)p.bias3)[n]);
  ((T *)p.C)[(int64_t)m * p.N + n] = from_f32<T>(silu_f(g) * u);
}

// --------------------------------------------------------------- bf16 MFMA
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_mfma(GemmProblem p0, GemmProblem p1, int tiles0, int ntm0,
                                                      int ntm1) {
  constexpr int WTM = BM / 2, WTN = BN / 2;     // wave tile
  constexpr int MT = WTM / 32, NT = WTN / 32;   // MFMA tiles per wave
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  static_assert(!SWI || NT % 2 == 0, "SwiGLU needs an even number of n tiles per wave");
  __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * LROW];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * LROW];

  int bid = blockIdx.x;
  const bool second = bid >= tiles0;
  const GemmProblem p = second ? p1 : p0;
  if (second) bid -= tiles0;
  const int ntm = second ? ntm1 : ntm0;
  const int tm = bid % ntm, tn = bid / ntm;
  const int m0 = tm * BM;
  // output columns covered by this workgroup: BN (or BN/2 SwiGLU outputs)
  const int n0 = tn * (SWI ? BN / 2 : BN);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int M = p.M, K = p.K;
  const bf16 *A = (const bf16 *)p.A;
  const bf16 *W = (const bf16 *)p.W;
  const bf16 *W3 = (const bf16 *)p.W3;

  // global -> register staging: 16-byte chunks, 8 chunks per 64-wide row
  constexpr int A_LD = BM * 8 / 256, B_LD = BN * 8 / 256;
  const int ck = (tid & 7) * 8;   // k offset of this thread's chunk
  const int rr = tid >> 3;        // first row (0..31), then +32 per load
  const bf16 *a_src[A_LD];
  const bf16 *b_src[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    int r = m0 + rr + 32 * i;
    r = r < M ? r : M - 1;
    a_src[i] = A + (int64_t)r * K + ck;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    int r = rr + 32 * i;  // row inside the B tile
    const bf16 *base;
    if constexpr (SWI) {
      base = r < BN / 2 ? W + (int64_t)(n0 + r) * K : W3 + (int64_t)(n0 + r - BN / 2) * K;
    } else {
      base = W + (int64_t)(n0 + r) * K;
    }
    b_src[i] = base + ck;
  }
  u32x4 ra[A_LD], rb[B_LD];
#define GEMM_GLOAD(k0)                                                              \
  do {                                                                              \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) ra[i] = *(const u32x4 *)(a_src[i] + (k0)); \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i) rb[i] = *(const u32x4 *)(b_src[i] + (k0)); \
  } while (0)
#define GEMM_LSTORE(buf)                                                                          \
  do {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) *(u32x4 *)&sA[buf][(rr + 32 * i) * LROW + ck] = ra[i]; \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i) *(u32x4 *)&sB[buf][(rr + 32 * i) * LROW + ck] = rb[i]; \
  } while (0)

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

  // LDS row of each MFMA tile's fragment for this lane
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  int a_row[MT], b_row[NT];
#pragma unroll
  for (int i = 0; i < MT; ++i) a_row[i] = wm * WTM + i * 32 + frow;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if constexpr (SWI) {
      constexpr int H = NT / 2;
      b_row[j] = (j < H ? wn * (WTN / 2) + j * 32 : BN / 2 + wn * (WTN / 2) + (j - H) * 32) + frow;
    } else {
      b_row[j] = wn * WTN + j * 32 + frow;
    }
  }

  const int KT = K / BK;
  GEMM_GLOAD(0);
  GEMM_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) GEMM_GLOAD((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[MT], fb[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[i] = *(const bf16x8 *)&sA[buf][a_row[i] * LROW + ks * 16 + fk];
#pragma unroll
      for (int j = 0; j < NT; ++j) fb[j] = *(const bf16x8 *)&sB[buf][b_row[j] * LROW + ks * 16 + fk];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) GEMM_LSTORE(buf ^ 1);
    __syncthreads();
  }
#undef GEMM_GLOAD
#undef GEMM_LSTORE

  // epilogue: lane holds column (lane & 31) and rows (r/4)*8 + (lane/32)*4 + r%4
  const int cl = lane & 31, rh = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + rh + (r & 3);
      if (m >= M) continue;
      if constexpr (SWI) {
        constexpr int H = NT / 2;
#pragma unroll
        for (int j = 0; j < H; ++j) {
          const int n = n0 + wn * (WTN / 2) + j * 32 + cl;
          epi_swiglu<bf16>(p, m, n, acc[i][j][r], acc[i][j + H][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int n = n0 + wn * WTN + j * 32 + cl;
          epi_store<EPI, bf16>(p, m, n, acc[i][j][r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------ fp32 (FMA)
// 64 x 64 tile, 256 threads, 4 x 4 outputs per thread, K step 16.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_simple(GemmProblem p0, GemmProblem p1, int tiles0, int ntm0,
                                                       int ntm1) {
  constexpr int T = 64, TK = 16;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  __shared__ float sA[TK][T + 1];
  __shared__ float sB[TK][T + 1];
  __shared__ float sB3[SWI ? TK : 1][T + 1];
  int bid = blockIdx.x;
  const bool second = bid >= tiles0;
  const GemmProblem p = second ? p1 : p0;
  if (second) bid -= tiles0;
  const int ntm = second ? ntm1 : ntm0;
  const int m0 = (bid % ntm) * T, n0 = (bid / ntm) * T;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const float *A = (const float *)p.A, *W = (const float *)p.W, *W3 = (const float *)p.W3;
  float acc[4][4] = {}, acc3[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += TK) {
    for (int e = threadIdx.x; e < T * TK; e += 256) {
      const int r = e / TK, k = e % TK;
      const int m = m0 + r, n = n0 + r, kk = k0 + k;
      sA[k][r] = (m < p.M && kk < p.K) ? A[(int64_t)m * p.K + kk] : 0.f;
      sB[k][r] = (n < p.N && kk < p.K) ? W[(int64_t)n * p.K + kk] : 0.f;
      if constexpr (SWI) sB3[k][r] = (n < p.N && kk < p.K) ? W3[(int64_t)n * p.K + kk] : 0.f;
    }
    __syncthreads();
    for (int k = 0; k < TK; ++k) {
      float a[4], b[4], b3[4];
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
      for (int j = 0; j < 4; ++j) {
        b[j] = sB[k][tx * 4 + j];
        if constexpr (SWI) b3[j] = sB3[k][tx * 4 + j];
      }
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if constexpr (SWI) acc3[i][j] = fmaf(a[i], b3[j], acc3[i][j]);
        }
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m >= p.M || n >= p.N) continue;
      if constexpr (SWI)
        epi_swiglu<float>(p, m, n, acc[i][j], acc3[i][j]);
      else
        epi_store<EPI, float>(p, m, n, acc[i][j]);
    }
}

template <int BM, int BN, int EPI>
hipError_t run_bf16(const GemmProblem *pr, int np, hipStream_t st) {
  const int wn = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  int ntm[2] = {0, 0}, tiles[2] = {0, 0};
  for (int i = 0; i < np; ++i) {
    ntm[i] = (pr[i].M + BM - 1) / BM;
    tiles[i] = pr[i].M > 0 ? ntm[i] * (pr[i].N / wn) : 0;
  }
  const int total = tiles[0] + tiles[1];
  if (total == 0) return hipSuccess;
  GemmProblem q1 = np > 1 ? pr[1] : pr[0];
  hipLaunchKernelGGL((gemm_bf16_mfma<BM, BN, EPI>), dim3(total), dim3(256), 0, st, pr[0], q1, tiles[0],
                     ntm[0] > 0 ? ntm[0] : 1, ntm[1] > 0 ? ntm[1] : 1);
  return hipGetLastError();
}

template <int EPI>
hipError_t run_f32(const GemmProblem *pr, int np, hipStream_t st) {
  int ntm[2] = {1, 1}, tiles[2] = {0, 0};
  for (int i = 0; i < np; ++i) {
    ntm[i] = (pr[i].M + 63) / 64;
    tiles[i] = pr[i].M > 0 ? ntm[i] * ((pr[i].N + 63) / 64) : 0;
    if (ntm[i] == 0) ntm[i] = 1;
  }
  const int total = tiles[0] + tiles[1];
  if (total == 0) return hipSuccess;
  GemmProblem q1 = np > 1 ? pr[1] : pr[0];
  hipLaunchKernelGGL((gemm_f32_simple<EPI>), dim3(total), dim3(256), 0, st, pr[0], q1, tiles[0], ntm[0], ntm[1]);
  return hipGetLastError();
}

}  // namespace

// The bf16 kernel needs K % 64 == 0 and N % 128 == 0 (N % 64 for SwiGLU
// outputs); the caller checks this.  M may be anything >= 0.
hipError_t launch_gemm(int epi, bool bf16_path, const GemmProblem *probs, int nprob, hipStream_t stream) {
  if (bf16_path) {
    switch (epi) {
      case EPI_STORE: return run_bf16<256, 128, EPI_STORE>(probs, nprob, stream);
      case EPI_STORE_F32: return run_bf16<256, 128, EPI_STORE_F32>(probs, nprob, stream);
      case EPI_GATED: return run_bf16<256, 128, EPI_GATED>(probs, nprob, stream);
      case EPI_SWIGLU: return run_bf16<256, 128, EPI_SWIGLU>(probs, nprob, stream);
    }
  } else {
    switch (epi) {
      case EPI_STORE: return run_f32<EPI_STORE>(probs, nprob, stream);
      case EPI_STORE_F32: return run_f32<EPI_STORE_F32>(probs, nprob, stream);
      case EPI_GATED: return run_f32<EPI_GATED>(probs, nprob, stream);
      case EPI_SWIGLU: return run_f32<EPI_SWIGLU>(probs, nprob, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lens

// GEMMs of the MM-DiT block: C[M, N] = A[M, K] . W[N, K]^T with fused
// epilogues (bias; gated residual h += gate * y; SwiGLU silu(y1) * y3).
//
// These are the per-stream Linear layers of each block (img_qkv / txt_qkv,
// to_out / to_add_out, img_mlp / txt_mlp w1 w3 w2 in the Lens-Turbo-3.8B-bf16
// article; the gated residual and gated MLP of the Lens blog's "Overview").
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation.  A
// workgroup of WM x WN waves computes a BM x BN tile (256 x 256 with 8
// waves, two per SIMD, for the large projections).  K advances in slabs of
// 32 that direct global->LDS loads drop into a ring of LDS stages, several
// slabs ahead of the MFMAs.  Both operands are K-contiguous, so every load
// and every LDS fragment read is a 16-byte vector.  The epilogue stages the
// accumulators through LDS and writes rows with 16-byte stores.  Image and
// text problems (different weights, different M) run in one grouped launch,
// in an order that keeps each XCD's tiles on shared A and W panels.
//
// fp32 path: a plain LDS-tiled FMA kernel with the same epilogues, used by
// the fp32 configuration (correctness, not speed).
#include "common.h"

namespace lens {

namespace {

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

// ------------------------------------------- bf16 MFMA, LDS-DMA pipeline
// Direct global->LDS loads (global_load_lds_dwordx4: each lane's 16 bytes
// land at M0 + 16 * lane, so one wave instruction fills 1 KB of LDS) into a
// ring of NSTAGE slabs of BK = 32, prefetching NSTAGE - 1 slabs ahead; no
// VGPRs hold staged data.  A slab row is 64 bytes (four 16-byte chunks); the
// chunk of row r at k-chunk c sits in slot c ^ ((r >> SWZ_SHIFT) & 3), which
// spreads the 32 rows one fragment read touches over all LDS banks.
namespace dma {
constexpr int DBK = 32;            // k per slab
constexpr int ROWB = DBK * 2;      // bytes per slab row
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r, int shift) { return (r >> shift) & 3; }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// lgkmcnt(0) only: this wave's LDS reads have returned
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }
}  // namespace dma

// Epilogue through LDS, one wm-slice (WTM rows) at a time: the waves of
// that slice park their fp32 accumulators in row-major order, then every
// thread applies the epilogue to 8 consecutive columns and writes them with
// 16-byte vector stores.  bcol[j]: tile column of accumulator tile j for
// this lane.  st must hold WTM * (BN + 4) floats; the caller's LDS is free.
template <int BM, int BN, int WM, int MT, int NT, int NTH, int EPI>
__device__ __forceinline__ void epilogue_lds(const GemmProblem &p, const f32x16 (&acc)[MT][NT], float *st, int m0,
                                             int n0, int wm, const int (&bcol)[NT], int lane, int tid) {
  constexpr int WTM = BM / WM;
  constexpr int EPI_LDW = BN + 4;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  const int M = p.M;
  const int rh = (lane >> 5) * 4;
#pragma unroll
  for (int h = 0; h < WM; ++h) {
    dma::wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            st[(i * 32 + (r >> 2) * 8 + rh + (r & 3)) * EPI_LDW + bcol[j]] = acc[i][j][r];
    }
    dma::wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    constexpr int OUTC = SWI ? BN / 2 : BN;      // output columns of the tile
    constexpr int TPR = OUTC / 8;                // threads per row
    constexpr int RPP = NTH / TPR;               // rows per pass
    const int c8 = (tid % TPR) * 8;
    const int n = n0 + c8;
    for (int rr = tid / TPR; rr < WTM; rr += RPP) {
      const int m = m0 + h * WTM + rr;
      if (m >= M) break;
      const float *src = st + rr * EPI_LDW + c8;
      float v[8];
      *(float4 *)&v[0] = *(const float4 *)src;
      *(float4 *)&v[4] = *(const float4 *)(src + 4);
      if constexpr (SWI) {
        float u[8];
        *(float4 *)&u[0] = *(const float4 *)(src + BN / 2);
        *(float4 *)&u[4] = *(const float4 *)(src + BN / 2 + 4);
        bf16x8 o;
        const bf16x8 b1 = p.bias ? *(const bf16x8 *)((const bf16 *)p.bias + n) : bf16x8{};
        const bf16x8 b3 = p.bias3 ? *(const bf16x8 *)((const bf16 *)p.bias3 + n) : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)(silu_f(v[e] + (float)b1[e]) * (u[e] + (float)b3[e]));
        *(bf16x8 *)((bf16 *)p.C + (int64_t)m * p.N + n) = o;
      } else {
        if (p.bias) {
          const bf16x8 bb = *(const bf16x8 *)((const bf16 *)p.bias + n);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += (float)bb[e];
        }
        if constexpr (EPI == EPI_STORE) {
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
          *(bf16x8 *)((bf16 *)p.C + (int64_t)m * p.N + n) = o;
        } else if constexpr (EPI == EPI_STORE_F32) {
          float *dst = (float *)p.C + (int64_t)m * p.N + n;
          *(float4 *)dst = *(float4 *)&v[0];
          *(float4 *)(dst + 4) = *(float4 *)&v[4];
        } else {
          const float *g = p.gate + (int64_t)(m / p.rows_per_gate) * p.gate_stride + n;
          float *dst = (float *)p.C + (int64_t)m * p.N + n;
          float4 h0 = *(float4 *)dst, h1 = *(float4 *)(dst + 4);
          const float4 g0 = *(const float4 *)g, g1 = *(const float4 *)(g + 4);
          h0.x += g0.x * v[0]; h0.y += g0.y * v[1]; h0.z += g0.z * v[2]; h0.w += g0.w * v[3];
          h1.x += g1.x * v[4]; h1.y += g1.y * v[5]; h1.z += g1.z * v[6]; h1.w += g1.w * v[7];
          *(float4 *)dst = h0;
          *(float4 *)(dst + 4) = h1;
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int NSTAGE, int SWZ, int EPI, int GM, bool XCD = true>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_dma(GemmProblem p0, GemmProblem p1, int tiles0,
                                                              int ntm0, int ntm1, int total_tiles) {
  using namespace dma;
  constexpr int NTH = 64 * WM * WN, NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  static_assert(!SWI || NT % 2 == 0, "SwiGLU needs an even number of n tiles per wave");
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
  // rows written by one wave instruction: 1 KB / 64 B = 16; per round of all waves: 16 * NW
  constexpr int ROWS_PER_ROUND = 16 * NW;
  constexpr int A_RND = BM / ROWS_PER_ROUND, B_RND = BN / ROWS_PER_ROUND;
  static_assert(A_RND * ROWS_PER_ROUND == BM && B_RND * ROWS_PER_ROUND == BN, "rows must split over waves");
  constexpr int LD_PER_STAGE = A_RND + B_RND;   // load instructions per thread per slab
  constexpr int EPI_LDW = BN + 4;                // fp32 row stride of the epilogue staging
  constexpr int EPI_BYTES = WTM * EPI_LDW * 4;
  constexpr int SMEM = NSTAGE * STAGE > EPI_BYTES ? NSTAGE * STAGE : EPI_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  // XCD-aware order: dispatch round-robins workgroups over the 8 XCDs, so
  // give XCD x a contiguous run of logical tiles (sharing its L2).
  int bid = blockIdx.x;
  if (XCD) {
    const int per = total_tiles / 8;
    if (bid < per * 8) bid = (bid % 8) * per + bid / 8;
  }
  const bool second = bid >= tiles0;
  const GemmProblem p = second ? p1 : p0;
  if (second) bid -= tiles0;
  const int ntm = second ? ntm1 : ntm0;
  // grouped order: GM m-tiles vary fastest inside a group, then n, so the
  // tiles an XCD runs together share GM panels of A and stream W panels
  const int ntn = (SWI ? p.N / (BN / 2) : p.N / BN);
  const int group = bid / (GM * ntn), first_m = group * GM;
  const int gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
  const int tm = first_m + (bid % (GM * ntn)) % gsz;
  const int tn = (bid % (GM * ntn)) / gsz;
  const int m0 = tm * BM;
  const int n0 = tn * (SWI ? BN / 2 : BN);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int M = p.M, K = p.K;
  const bf16 *A = (const bf16 *)p.A;
  const bf16 *W = (const bf16 *)p.W;
  const bf16 *W3 = (const bf16 *)p.W3;

  // this lane's source rows/chunks for each load instruction of a slab
  const int lrow = lane >> 2, lslot = lane & 3;
  const bf16 *a_src[A_RND];
  const bf16 *b_src[B_RND];
#pragma unroll
  for (int i = 0; i < A_RND; ++i) {
    const int r = i * ROWS_PER_ROUND + wave * 16 + lrow;
    int gr = m0 + r;
    gr = gr < M ? gr : M - 1;
    a_src[i] = A + (int64_t)gr * K + (lslot ^ swz(r, SWZ)) * 8;
  }
#pragma unroll
  for (int i = 0; i < B_RND; ++i) {
    const int r = i * ROWS_PER_ROUND + wave * 16 + lrow;
    const bf16 *base;
    if constexpr (SWI) {
      base = r < BN / 2 ? W + (int64_t)(n0 + r) * K : W3 + (int64_t)(n0 + r - BN / 2) * K;
    } else {
      base = W + (int64_t)(n0 + r) * K;
    }
    b_src[i] = base + (lslot ^ swz(r, SWZ)) * 8;
  }
  // LDS destination (wave-uniform) of instruction i inside a stage
  const int a_dst0 = wave * 16 * ROWB, b_dst0 = A_BYTES + wave * 16 * ROWB;

#define DMA_ISSUE(kt_)                                                                                   \
  do {                                                                                                   \
    char *sb_ = smem + ((kt_) % NSTAGE) * STAGE;                                                         \
    const int k0_ = (kt_) * DBK;                                                                         \
    _Pragma("unroll") for (int i = 0; i < A_RND; ++i) __builtin_amdgcn_global_load_lds(                  \
        (const void *)(a_src[i] + k0_), (lds_void *)(sb_ + a_dst0 + i * ROWS_PER_ROUND * ROWB), 16, 0, 0); \
    _Pragma("unroll") for (int i = 0; i < B_RND; ++i) __builtin_amdgcn_global_load_lds(                  \
        (const void *)(b_src[i] + k0_), (lds_void *)(sb_ + b_dst0 + i * ROWS_PER_ROUND * ROWB), 16, 0, 0); \
  } while (0)

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

  // fragment rows for this lane
  const int frow = lane & 31, hl = lane >> 5;
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

  const int KT = K / DBK;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < KT) DMA_ISSUE(s);

  for (int kt = 0; kt < KT; ++kt) {
    // slabs issued after kt that may stay in flight
    const int ahead = (KT - 1 - kt) < (NSTAGE - 2) ? (KT - 1 - kt) : (NSTAGE - 2);
    if (ahead >= 2) wait_vm<2 * LD_PER_STAGE>();
    else if (ahead == 1) wait_vm<LD_PER_STAGE>();
    else wait_vm<0>();
    // Barrier without a memory fence: the waits above cover this wave's
    // slab loads and LDS reads, and a fence would drain every prefetch.
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if (kt + NSTAGE - 1 < KT) DMA_ISSUE(kt + NSTAGE - 1);
    const char *sb = smem + (kt % NSTAGE) * STAGE;
#pragma unroll
    for (int ks = 0; ks < DBK / 16; ++ks) {
      const int c = ks * 2 + hl;   // 16-byte k-chunk this lane reads
      bf16x8 fa[MT], fb[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        fa[i] = *(const bf16x8 *)(sb + a_row[i] * ROWB + ((c ^ swz(a_row[i], SWZ)) << 4));
#pragma unroll
      for (int j = 0; j < NT; ++j)
        fb[j] = *(const bf16x8 *)(sb + A_BYTES + b_row[j] * ROWB + ((c ^ swz(b_row[j], SWZ)) << 4));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

#undef DMA_ISSUE
  int bcol[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) bcol[j] = b_row[j] - frow + (lane & 31);
  epilogue_lds<BM, BN, WM, MT, NT, NTH, EPI>(p, acc, (float *)smem, m0, n0, wm, bcol, lane, tid);
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

template <int BM, int BN, int WM, int WN, int NSTAGE, int SWZ, int EPI, int GM = 4, bool XCD = true>
hipError_t run_dma(const GemmProblem *pr, int np, hipStream_t st) {
  const int wn = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  int ntm[2] = {0, 0}, tiles[2] = {0, 0};
  for (int i = 0; i < np; ++i) {
    ntm[i] = (pr[i].M + BM - 1) / BM;
    tiles[i] = pr[i].M > 0 ? ntm[i] * (pr[i].N / wn) : 0;
  }
  const int total = tiles[0] + tiles[1];
  if (total == 0) return hipSuccess;
  GemmProblem q1 = np > 1 ? pr[1] : pr[0];
  hipLaunchKernelGGL((gemm_bf16_dma<BM, BN, WM, WN, NSTAGE, SWZ, EPI, GM, XCD>), dim3(total), dim3(64 * WM * WN), 0, st,
                     pr[0], q1, tiles[0], ntm[0] > 0 ? ntm[0] : 1, ntm[1] > 0 ? ntm[1] : 1, total);
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

// bf16 tile choice: 256 x 256 tiles (8 waves, 2 per SIMD) unless that grid
// would leave the chip under-filled, then 128 x 256 tiles; N not a
// multiple of 256 (the 128-wide velocity projection) takes 256 x 128.
// The caller guarantees K % 32 == 0 and N % 128 == 0 (SwiGLU: N % 128 == 0
// output columns, i.e. 256 rows of w1 | w3 per tile).  M may be anything.
template <int EPI>
hipError_t dispatch_bf16(const GemmProblem *pr, int np, hipStream_t st) {
  constexpr bool SWI = EPI == EPI_SWIGLU;
  const int outc = SWI ? 128 : 256;   // output columns of a 256-wide tile
  bool n256 = true;
  int tiles256 = 0;
  for (int i = 0; i < np; ++i) {
    if (pr[i].N % outc) n256 = false;
    tiles256 += ((pr[i].M + 255) / 256) * (pr[i].N / outc);
  }
  if (!n256) return run_dma<256, 128, 4, 2, 4, 2, EPI>(pr, np, st);
  if (tiles256 < 200) return run_dma<128, 256, 2, 4, 4, 2, EPI>(pr, np, st);
  if (SWI) return run_dma<256, 256, 2, 4, 3, 2, EPI>(pr, np, st);
  return run_dma<256, 256, 2, 4, 4, 2, EPI>(pr, np, st);
}

hipError_t launch_gemm(int epi, bool bf16_path, const GemmProblem *probs, int nprob, hipStream_t stream) {
  if (bf16_path) {
    switch (epi) {
      case EPI_STORE: return dispatch_bf16<EPI_STORE>(probs, nprob, stream);
      case EPI_STORE_F32: return dispatch_bf16<EPI_STORE_F32>(probs, nprob, stream);
      case EPI_GATED: return dispatch_bf16<EPI_GATED>(probs, nprob, stream);
      case EPI_SWIGLU: return dispatch_bf16<EPI_SWIGLU>(probs, nprob, stream);
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

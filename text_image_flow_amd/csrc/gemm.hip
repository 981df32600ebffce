// GEMMs of the MM-DiT block: C[M, N] = A[M, K] . W[N, K]^T with fused
// epilogues (bias; gated residual h += gate * y; SwiGLU silu(y1) * y3).
//
// These are the per-stream Linear layers of each block (img_qkv / txt_qkv,
// to_out / to_add_out, img_mlp / txt_mlp w1 w3 w2 in the Lens-Turbo-3.8B-bf16
// article; the gated residual and gated MLP of the Lens blog's "Overview").
//
// bf16 path (gemm_bf16): v_mfma_f32_32x32x16_bf16 (gfx950), fp32
// accumulation, one persistent workgroup per CU.
//  * Tiles are BM x BN (256 x 256 for the large projections) computed by
//    WM x WN waves.  Image and text problems (different weights and M, same
//    N and K) share one launch; the tile order groups GM m-tiles so that the
//    tiles an XCD runs together share A and W panels, and workgroup b (which
//    the dispatcher places on XCD b % 8) walks a contiguous run of it.
//  * K advances in slabs 64 deep, so every slab row is one whole 128-byte
//    line: the address path serves a wave instruction covering 8 full lines
//    much faster than one covering 16 half lines.  Direct global->LDS loads
//    (each lane's 16 bytes land at M0 + 16 * lane; no VGPR holds staged data)
//    fill two rings, three A stages and two W stages (160 KB).  They are raw
//    buffer loads (buffer_load_dwordx4 ... lds): each lane keeps one 32-bit
//    row offset and the slab's k offset rides in the scalar offset, so a
//    load needs no address arithmetic (64-bit global loads are the fallback
//    for operands of 2 GiB or more).  Chunk c of
//    row r sits in slot c ^ ((r >> 1) & 7), so any 16 consecutive rows of a
//    fragment read hit all 64 banks.
//  * The slab stream runs on across tile boundaries, so the next tile's first
//    slabs load while this tile's epilogue runs.  Fragments are
//    double-buffered (step ks + 1's LDS reads go out before step ks's
//    MFMAs) and a slab's loads are spread over the four k steps.
//  * The epilogue works from registers: the MFMAs take the weight fragment as
//    the first operand, so each lane's accumulators hold one token and runs
//    of 4 consecutive features (C^T layout); one permlane32 swap per dword
//    makes 8 consecutive bf16 per lane for a 16-byte store.  Biases arrive
//    through scalar loads, which leave the vector-memory counter to the slabs.
//
// MX fp8 path (same kernel, F8 = true; the low-precision block projections
// of the Lens-3.8B-4bit article, section 4, as MX-style fp8 with a
// non-saturating scale): e4m3 operands
// with one E8M0 scale per 32 along K, v_mfma_scale_f32_32x32x64_f8f6f4.
//  * A slab is 128 k deep (still one 128-byte line per row), two MFMA k
//    steps; each lane's scale dword holds its row's 4 block scales of the
//    slab, loaded one slab ahead between the slab's W and A parts.
//  * A fragments are read one row tile ahead, W fragments one k step ahead,
//    and each MFMA is held in place by an empty asm on its accumulator.
//  * EPI_SWIGLU_MX writes the SwiGLU output itself as MX fp8 (the input of
//    the w2 projection).
//
// fp32 path: a plain LDS-tiled FMA kernel with the same epilogues, used by
// the fp32 configuration (correctness, not speed).
#include <stdlib.h>

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

namespace gk {
constexpr int RBK = 64;            // k per slab
constexpr int RROW = RBK * 2;      // bytes per slab row (one 128-byte line)
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(4))) unsigned *cptr;

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// 16 bytes per lane from base + voff + soff into LDS at M0 + 16 * lane, as a
// raw buffer load (bounds = bytes)
__device__ __forceinline__ void buffer_lds16(const void *base, int bytes, lds_void *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, bytes, 0x00020000),
                                           dst, 16, voff, soff, 0, 0);
}
// lgkmcnt(0) only: this wave's LDS reads have returned
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ unsigned pack_bf2(float a, float b) {
  const bf16x2 t = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(unsigned, t);
}

// Tile t of the grouped launch -> problem (second), first row and column.
__device__ __forceinline__ void tile_coords(int t, int tiles0, int ntm0, int ntm1, int ntn, int gm, int bm, int outc,
                                            bool &second, int &m0, int &n0) {
  second = t >= tiles0;
  const int b = second ? t - tiles0 : t;
  const int ntm = second ? ntm1 : ntm0;
  const int group = b / (gm * ntn), first_m = group * gm;
  const int gsz = (ntm - first_m) < gm ? (ntm - first_m) : gm;
  const int r = b % (gm * ntn);
  m0 = (first_m + r % gsz) * bm;
  n0 = (r / gsz) * outc;
}

// Two runs of 4 accumulators as bf16 pairs (features 8q .. 8q+3 on lanes
// 0-31 and 8q+4 .. 8q+7 on lanes 32-63, then the same for q+1): after the
// swaps lanes 0-31 hold features 8q .. 8q+7 and lanes 32-63 8q+8 .. 8q+15.
__device__ __forceinline__ u32x4 pair_runs(unsigned x0, unsigned x1, unsigned y0, unsigned y1) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
  return u32x4{s0[0], s1[0], s0[1], s1[1]};
}
}  // namespace gk

// Epilogue of one output tile from the accumulators of one wave (WTM x WTN
// of the tile, row tiles of 32 x 32): bias, then the epilogue's own work,
// stored straight from registers.  The MFMAs take the weight fragment
// first, so a lane's accumulators hold one token and runs of 4 consecutive
// features (C^T layout); one permlane32 swap per dword makes 8 consecutive
// bf16 per lane for a 16-byte store.  Biases arrive through scalar loads,
// which leave the vector-memory counter to the slab loads.
template <int EPI, int MT, int NT, int WTM, int WTN>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[MT][NT], const GemmProblem &p0, const GemmProblem &p1,
                                           const QkvOut &qo, int ct, int tiles0, int ntm0, int ntm1, int ntn, int GM,
                                           int BM, int OUTC, int wm, int wn, int lane) {
  using namespace gk;
  constexpr bool SWI = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX);
  constexpr int H = SWI ? NT / 2 : NT;
  const int frow = lane & 31, hl = lane >> 5;
  bool sec;
  int m0, n0;
  tile_coords(ct, tiles0, ntm0, ntm1, ntn, GM, BM, OUTC, sec, m0, n0);
  const int M = sec ? p1.M : p0.M, N = p0.N;
  void *C = sec ? p1.C : p0.C;
  const void *bias = sec ? p1.bias : p0.bias;
  // wave's first output feature; lane holds features fw + j*32 + 8q + 4*hl + e
  const int fw = n0 + wn * (WTN / (SWI ? 2 : 1));
  const void *bias3 = SWI ? (sec ? p1.bias3 : p0.bias3) : nullptr;
  // Biases of one 32-feature column group (16 dwords) per scalar load;
  // this lane's 4 bf16 for (j, q) are dwords 4q + 2*hl + {0, 1}.
#define LOAD_BIAS16(ptr_, j_, arr_)                                                        \
do {                                                                                     \
  if (ptr_) {                                                                            \
    const cptr bp_ = (cptr)((const bf16 *)(ptr_) + fw + (j_) * 32);                      \
    _Pragma("unroll") for (int k = 0; k < 16; ++k) arr_[k] = bp_[k];                     \
  } else {                                                                               \
    _Pragma("unroll") for (int k = 0; k < 16; ++k) arr_[k] = 0;                          \
  }                                                                                      \
} while (0)
#define BIAS4(arr_, j_, q_, out_)                                                          \
do {                                                                                     \
  const unsigned lo_ = hl ? arr_[4 * (q_) + 2] : arr_[4 * (q_)];                         \
  const unsigned hi_ = hl ? arr_[4 * (q_) + 3] : arr_[4 * (q_) + 1];                     \
  out_[0] = bf_lo(lo_);                                                            \
  out_[1] = bf_hi(lo_);                                                            \
  out_[2] = bf_lo(hi_);                                                            \
  out_[3] = bf_hi(hi_);                                                            \
} while (0)
  if constexpr (EPI == EPI_QKV) {
    // This wave's 64 features are one head of q, k or v.  Lanes l and
    // l ^ 32 hold the two halves of a token's head: features
    // j*32 + 8q + 4*hl + e.
    const int D = qo.H * 64;
    const int sect = fw / D, hh = (fw - sect * D) >> 6;
    bf16 *const dst = (bf16 *)(sect == 0 ? qo.Q : sect == 1 ? qo.K : qo.V);
    const void *gain = sect == 0 ? qo.q_gain[sec ? 1 : 0] : qo.k_gain[sec ? 1 : 0];
    const int rps = sec ? qo.S_txt : qo.S_img, joff = sec ? qo.S_img : 0;
    const float osc = sect == 0 ? qo.q_scale : 1.0f;
    unsigned bw[2][16], gw[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      LOAD_BIAS16(bias, j, bw[j]);
      if (sect < 2) {
        const cptr gp_ = (cptr)((const bf16 *)gain + j * 32);
#pragma unroll
        for (int k = 0; k < 16; ++k) gw[j][k] = gp_[k];
      }
    }
    // Two passes, so that no wait for the RoPE table stands behind stores:
    // first every row tile is normalised, rotated and packed in registers
    // (its 8 table loads issued together), then all of them are stored.
    u32x4 packed[MT][2][2];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + wm * WTM + i * 32 + frow;
      const int mc = m < M ? m : 0;
      const int bsmp = mc / rps, joint = joff + (mc - bsmp * rps);
      float y[2][4][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float b[4];
          BIAS4(bw[j], j, q, b);
#pragma unroll
          for (int e = 0; e < 4; ++e) y[j][q][e] = acc[i][j][4 * q + e] + b[e];
        }
      if (sect < 2) {
        // this lane's rotation pairs j*16 + 4q + 2hl and the next one, as
        // float4 (cos, sin, cos, sin) index j*8 + 2q + hl of the token's row
        const float4 *rope = (const float4 *)(qo.rope + (int64_t)joint * 32);
        float4 cs[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) cs[j][q] = rope[j * 8 + 2 * q + hl];
        // RMSNorm over the head (the partner lane holds the other half)
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = fmaf(y[j][q][e], y[j][q][e], ss);
        const auto sw_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        const float r = rsqrtf((__uint_as_float(sw_[0]) + __uint_as_float(sw_[1])) / 64.f + qo.eps);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float g[4];
            BIAS4(gw[j], j, q, g);
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const float c = e ? cs[j][q].z : cs[j][q].x, sn = e ? cs[j][q].w : cs[j][q].y;
              const float a0 = y[j][q][e] * r * g[e], a1 = y[j][q][e + 1] * r * g[e + 1];
              y[j][q][e] = (a0 * c - a1 * sn) * osc;
              y[j][q][e + 1] = (a0 * sn + a1 * c) * osc;
            }
          }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        unsigned pk[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          pk[q][0] = pack_bf2(y[j][q][0], y[j][q][1]);
          pk[q][1] = pack_bf2(y[j][q][2], y[j][q][3]);
        }
#pragma unroll
        for (int q = 0; q < 4; q += 2) packed[i][j][q / 2] = pair_runs(pk[q][0], pk[q][1], pk[q + 1][0], pk[q + 1][1]);
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + wm * WTM + i * 32 + frow;
      if (m < M) {
        const int bsmp = m / rps, joint = joff + (m - bsmp * rps);
        bf16 *row = dst + (((int64_t)bsmp * qo.H + hh) * qo.S_pad + joint) * 64;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; q += 2) *(u32x4 *)(row + j * 32 + 8 * q + 8 * hl) = packed[i][j][q / 2];
      }
    }
  } else if constexpr (EPI == EPI_GATED || EPI == EPI_STORE_F32) {
    // fp32 outputs.  Per row tile, every load (gate and h rows: 16 float4)
    // goes out before the first use, so the tile waits once, not once per
    // float4 behind the stores before it; rows past M load row 0 and store
    // nothing.
    unsigned bw[H][16];
#pragma unroll
    for (int j = 0; j < H; ++j) LOAD_BIAS16(bias, j, bw[j]);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + wm * WTM + i * 32 + frow;
      const bool ok = m < M;
      const int mc = ok ? m : 0;
      float *hrow = (float *)C + (int64_t)mc * N + fw + 4 * hl;
      float4 g4[H][4], h4[H][4];
      if constexpr (EPI == EPI_GATED) {
        const float *g = sec ? p1.gate : p0.gate;
        const int rpg = sec ? p1.rows_per_gate : p0.rows_per_gate;
        const int gst = sec ? p1.gate_stride : p0.gate_stride;
        const float *grow = g + (int64_t)(mc / rpg) * gst + fw + 4 * hl;
#pragma unroll
        for (int j = 0; j < H; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            g4[j][q] = *(const float4 *)(grow + j * 32 + 8 * q);
            h4[j][q] = *(const float4 *)(hrow + j * 32 + 8 * q);
          }
      }
#pragma unroll
      for (int j = 0; j < H; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float b[4];
          BIAS4(bw[j], j, q, b);
          float4 y;
          y.x = acc[i][j][4 * q + 0] + b[0];
          y.y = acc[i][j][4 * q + 1] + b[1];
          y.z = acc[i][j][4 * q + 2] + b[2];
          y.w = acc[i][j][4 * q + 3] + b[3];
          if constexpr (EPI == EPI_GATED) {
            float4 o = h4[j][q];
            o.x += g4[j][q].x * y.x;
            o.y += g4[j][q].y * y.y;
            o.z += g4[j][q].z * y.z;
            o.w += g4[j][q].w * y.w;
            y = o;
          }
          if (ok) *(float4 *)(hrow + j * 32 + 8 * q) = y;
        }
    }
  } else {
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + wm * WTM + i * 32 + frow;
    const bool ok = m < M;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int f0 = fw + j * 32 + 4 * hl;     // + 8q
      unsigned bw[16], bw3[16];
      LOAD_BIAS16(bias, j, bw);
      if constexpr (SWI) LOAD_BIAS16(bias3, j, bw3);
      if constexpr (EPI == EPI_SWIGLU_MX) {
        // one MX block = this (token, 32-feature group): 16 values here,
        // 16 on the partner lane l ^ 32; after the swaps lanes 0-31 hold
        // bytes 0-15 of the block and lanes 32-63 bytes 16-31
        float b[4], b3[4], y[4][4], am = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          BIAS4(bw, j, q, b);
          BIAS4(bw3, j, q, b3);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[q][e] = silu_f(acc[i][j][4 * q + e] + b[e]) * (acc[i][j + H][4 * q + e] + b3[e]);
            am = fmaxf(am, fabsf(y[q][e]));
          }
        }
        const auto sa_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(am), __float_as_uint(am), false, false);
        const int ex = mx_exponent(fmaxf(__uint_as_float(sa_[0]), __uint_as_float(sa_[1])));
        unsigned d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = mx_pack4(y[q][0], y[q][1], y[q][2], y[q][3], ex);
        const auto s0 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
        if (ok) {
          const int64_t f = fw + j * 32;
          *(u32x4 *)((unsigned char *)C + (int64_t)m * N + f + 16 * hl) = u32x4{s0[0], s0[1], s1[0], s1[1]};
          if (hl == 0) ((unsigned char *)(sec ? p1.C_scale : p0.C_scale))[mx_scale_index(m, f / 32, M)] =
              (unsigned char)(ex + 127);
        }
      } else {
        unsigned pk[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float b[4], y[4];
          BIAS4(bw, j, q, b);
          if constexpr (SWI) {
            float b3[4];
            BIAS4(bw3, j, q, b3);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              y[e] = silu_f(acc[i][j][4 * q + e] + b[e]) * (acc[i][j + H][4 * q + e] + b3[e]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * q + e] + b[e];
          }
          pk[q][0] = pack_bf2(y[0], y[1]);
          pk[q][1] = pack_bf2(y[2], y[3]);
        }
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
          const u32x4 o = pair_runs(pk[q][0], pk[q][1], pk[q + 1][0], pk[q + 1][1]);
          if (ok) *(u32x4 *)((bf16 *)C + (int64_t)m * N + (f0 - 4 * hl) + 8 * q + 8 * hl) = o;
        }
      }
    }
  }
  }
#undef BIAS4
#undef LOAD_BIAS16
}

template <int BM, int BN, int WM, int WN, int EPI, int GM, bool BUF = false, bool F8 = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16(GemmProblem p0, GemmProblem p1, int tiles0, int ntm0,
                                                          int ntm1, int total_tiles, int per_xcd, QkvOut qo) {
  using namespace gk;
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr bool SWI = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX);
  constexpr int OUTC = SWI ? BN / 2 : BN;
  constexpr int H = SWI ? NT / 2 : NT;          // output sub-tiles per wave along n
  static_assert(!SWI || NT % 2 == 0, "SwiGLU needs an even number of n tiles per wave");
  static_assert(EPI != EPI_QKV || WTN == 64, "QKV epilogue: one head (64 features) per wave");
  constexpr int NA = 3, NB = 2;                 // ring depths: A two slabs ahead, W one
  constexpr int A_UNIT = BM * RROW, B_UNIT = BN * RROW;
  constexpr int ROWS_PER_ROUND = 8 * NW;        // one wave instruction: 8 rows x 128 B
  constexpr int LDA = BM / ROWS_PER_ROUND, LDB = BN / ROWS_PER_ROUND;
  static_assert(LDA * ROWS_PER_ROUND == BM && LDB * ROWS_PER_ROUND == BN, "rows must split over waves");
  static_assert(!F8 || BUF, "fp8 operands use buffer loads");
  constexpr int ES = F8 ? 1 : 2;                // bytes per element
  constexpr int SLAB_K = RROW / ES;             // k per slab (one 128-byte line per row)
  constexpr int KS = SLAB_K / (F8 ? 64 : 16);   // MFMA k steps per slab
  static_assert(LDB % (KS / 2) == 0 && LDA % (KS / 2) == 0, "load parts must split over half the steps");
  constexpr int PB = LDB / (KS / 2), PA = LDA / (KS / 2);
  constexpr int SMEM = NA * A_UNIT + NB * B_UNIT;
  static_assert(SMEM <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  char *const a_ring = smem;
  char *const b_ring = smem + NA * A_UNIT;

  // workgroup b sits on XCD b % 8; the XCD's tiles are one contiguous run
  // of the grouped order, dealt round-robin to its workgroups
  const int xcd = blockIdx.x & 7, nslot = gridDim.x >> 3;
  const int t_end = min((xcd + 1) * per_xcd, total_tiles);
  const int t_first = xcd * per_xcd + (blockIdx.x >> 3);
  if (t_first >= t_end) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int ntn = p0.N / OUTC;
  const int K = p0.K, KT = K / SLAB_K;
  const int lrow = lane >> 3, lslot = lane & 7;
  const int dst0 = wave * 8 * RROW;             // wave's rows inside a round

  // ---- two load streams (A and W), each with its own tile / slab cursor
  const bf16 *a_src[LDA];
  const bf16 *b_src[LDB];
  // BUF: buffer loads; per-lane 32-bit byte offsets, the slab's k offset in
  // the scalar offset, one resource per operand (two for w1 | w3)
  int a_off[LDA], b_off[LDB];
  const void *a_base = nullptr, *b_base = nullptr, *b3_base = nullptr;
  int a_bytes = 0, b_bytes = 0;
  int at = t_first, akt = 0, apos = 0;
  int bt = t_first, bkt = 0, bpos = 0;
#define A_SETUP(t_)                                                                                       \
  do {                                                                                                    \
    bool sec_;                                                                                            \
    int m0_, n0_;                                                                                         \
    tile_coords(t_, tiles0, ntm0, ntm1, ntn, GM, BM, OUTC, sec_, m0_, n0_);                               \
    const bf16 *A_ = (const bf16 *)(sec_ ? p1.A : p0.A);                                                  \
    const int M_ = sec_ ? p1.M : p0.M;                                                                    \
    _Pragma("unroll") for (int i = 0; i < LDA; ++i) {                                                     \
      const int r = i * ROWS_PER_ROUND + wave * 8 + lrow;                                                 \
      const int gr = m0_ + r < M_ ? m0_ + r : M_ - 1;                                                     \
      if constexpr (BUF) a_off[i] = (int)__umul24(gr, K * ES) + (lslot ^ swz(r)) * 16;                    \
      else a_src[i] = A_ + (int64_t)gr * K + (lslot ^ swz(r)) * 8;                                        \
    }                                                                                                     \
    if constexpr (BUF) {                                                                                  \
      a_base = A_;                                                                                        \
      a_bytes = M_ * K * ES;                                                                              \
    }                                                                                                     \
  } while (0)
#define B_SETUP(t_)                                                                                       \
  do {                                                                                                    \
    bool sec_;                                                                                            \
    int m0_, n0_;                                                                                         \
    tile_coords(t_, tiles0, ntm0, ntm1, ntn, GM, BM, OUTC, sec_, m0_, n0_);                               \
    const bf16 *W_ = (const bf16 *)(sec_ ? p1.W : p0.W);                                                  \
    const bf16 *W3_ = (const bf16 *)(sec_ ? p1.W3 : p0.W3);                                               \
    const int N_ = p0.N;                                                                                  \
    _Pragma("unroll") for (int i = 0; i < LDB; ++i) {                                                     \
      const int r = i * ROWS_PER_ROUND + wave * 8 + lrow;                                                 \
      if constexpr (BUF) {                                                                                \
        const int wr_ = SWI && r >= BN / 2 ? r - BN / 2 : r;                                              \
        b_off[i] = (int)__umul24(n0_ + wr_, K * ES) + (lslot ^ swz(r)) * 16;                              \
      } else {                                                                                            \
        const bf16 *base_;                                                                                \
        if constexpr (SWI) {                                                                              \
          base_ = r < BN / 2 ? W_ + (int64_t)(n0_ + r) * K : W3_ + (int64_t)(n0_ + r - BN / 2) * K;       \
        } else {                                                                                          \
          base_ = W_ + (int64_t)(n0_ + r) * K;                                                            \
        }                                                                                                 \
        b_src[i] = base_ + (lslot ^ swz(r)) * 8;                                                          \
      }                                                                                                   \
    }                                                                                                     \
    if constexpr (BUF) {                                                                                  \
      b_base = W_;                                                                                        \
      b3_base = W3_;                                                                                      \
      b_bytes = N_ * K * ES;                                                                              \
    }                                                                                                     \
  } while (0)
// one load instruction (part i) of the current A / W slab, and the cursor
// step once all parts of the slab are out
#define ISSUE_A_PART(i_)                                                                                   \
  do {                                                                                                     \
    lds_void *d_ = (lds_void *)(a_ring + apos * A_UNIT + dst0 + (i_) * ROWS_PER_ROUND * RROW);             \
    if constexpr (BUF)                                                                                     \
      buffer_lds16(a_base, a_bytes, d_, a_off[i_], akt * RROW);                                            \
    else                                                                                                   \
      __builtin_amdgcn_global_load_lds((const void *)(a_src[i_] + akt * RBK), d_, 16, 0, 0);               \
  } while (0)
#define ISSUE_B_PART(i_)                                                                                   \
  do {                                                                                                     \
    lds_void *d_ = (lds_void *)(b_ring + bpos * B_UNIT + dst0 + (i_) * ROWS_PER_ROUND * RROW);             \
    if constexpr (BUF) {                                                                                   \
      const void *bb_ = SWI && (i_) * ROWS_PER_ROUND >= BN / 2 ? b3_base : b_base;                        \
      buffer_lds16(bb_, b_bytes, d_, b_off[i_], bkt * RROW);                                               \
    } else {                                                                                               \
      __builtin_amdgcn_global_load_lds((const void *)(b_src[i_] + bkt * RBK), d_, 16, 0, 0);               \
    }                                                                                                      \
  } while (0)
#define STEP_A()                                                                                           \
  do {                                                                                                     \
    apos = apos + 1 == NA ? 0 : apos + 1;                                                                  \
    ++a_issued;                                                                                            \
    if (++akt == KT) {                                                                                     \
      akt = 0;                                                                                             \
      at += nslot;                                                                                         \
      if (at < t_end) A_SETUP(at);                                                                         \
    }                                                                                                      \
  } while (0)
#define STEP_B()                                                                                           \
  do {                                                                                                     \
    bpos = bpos + 1 == NB ? 0 : bpos + 1;                                                                  \
    if (++bkt == KT) {                                                                                     \
      bkt = 0;                                                                                             \
      bt += nslot;                                                                                         \
      if (bt < t_end) B_SETUP(bt);                                                                         \
    }                                                                                                      \
  } while (0)
#define ISSUE_A()                                                                                          \
  do {                                                                                                     \
    if (at < t_end) {                                                                                      \
      _Pragma("unroll") for (int i = 0; i < LDA; ++i) ISSUE_A_PART(i);                                     \
      STEP_A();                                                                                            \
    }                                                                                                      \
  } while (0)
#define ISSUE_B()                                                                                          \
  do {                                                                                                     \
    if (bt < t_end) {                                                                                      \
      _Pragma("unroll") for (int i = 0; i < LDB; ++i) ISSUE_B_PART(i);                                     \
      STEP_B();                                                                                            \
    }                                                                                                      \
  } while (0)

  // Issue order: A0 W0 A1, then in iteration k W(k+1) and after it A(k+2).
  // So when slab k is computed, W(k) is the newest W slab issued and at most
  // A(k+1) followed it (epilogue stores in between only make the wait
  // stricter).
  const int frow = lane & 31, hl = lane >> 5;
  int a_row[MT], b_row[NT];
#pragma unroll
  for (int i = 0; i < MT; ++i) a_row[i] = wm * WTM + i * 32 + frow;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if constexpr (SWI) {
      b_row[j] = (j < H ? wn * (WTN / 2) + j * 32 : BN / 2 + wn * (WTN / 2) + (j - H) * 32) + frow;
    } else {
      b_row[j] = wn * WTN + j * 32 + frow;
    }
  }

  // fp8 scales, stored slab-major ([K / 128][rows][4] E8M0 bytes): per
  // fragment row one dword = its 4 block scales of a slab, and the 32 rows of
  // a row tile are 128 consecutive bytes, so one load instruction touches one
  // cache line.  Loaded one slab ahead by raw buffer loads (a 32-bit row
  // offset per fragment, slab * rows * 4 in the scalar offset).  SC_SETUP
  // points the resources and offsets at tile t, SC_LOAD(slab) loads one
  // slab's dwords (raw; the lane-half shift happens at use).
  int so_a[F8 ? MT : 1], so_w[F8 ? NT : 1];
  unsigned s_a[F8 ? MT : 1], s_w[F8 ? NT : 1], n_a[F8 ? MT : 1], n_w[F8 ? NT : 1];
  int sa_step = 0, sw_step = 0;              // bytes per slab of the A / W scale arrays
  __amdgpu_buffer_rsrc_t rs_a, rs_w, rs_w3;
#define SC_SETUP(t_)                                                                                      \
  do {                                                                                                    \
    bool sec_;                                                                                            \
    int m0_, n0_;                                                                                         \
    tile_coords(t_, tiles0, ntm0, ntm1, ntn, GM, BM, OUTC, sec_, m0_, n0_);                               \
    const GemmProblem &pp_ = sec_ ? p1 : p0;                                                              \
    const int kb_ = K / 32;                                                                               \
    rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)pp_.A_scale, (short)0, pp_.M * kb_, 0x00020000);     \
    rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)pp_.W_scale, (short)0, pp_.N * kb_, 0x00020000);     \
    rs_w3 = __builtin_amdgcn_make_buffer_rsrc((void *)(SWI ? pp_.W3_scale : pp_.W_scale), (short)0,       \
                                              pp_.N * kb_, 0x00020000);                                   \
    sa_step = pp_.M * 4;                                                                                  \
    sw_step = pp_.N * 4;                                                                                  \
    _Pragma("unroll") for (int i = 0; i < MT; ++i) so_a[i] = min(m0_ + a_row[i], pp_.M - 1) * 4;          \
    _Pragma("unroll") for (int j = 0; j < NT; ++j) {                                                      \
      const bool third_ = SWI && b_row[j] >= BN / 2;                                                      \
      so_w[j] = (n0_ + (third_ ? b_row[j] - BN / 2 : b_row[j])) * 4;                                      \
    }                                                                                                     \
  } while (0)
#define SC_LOAD(slab_)                                                                                    \
  do {                                                                                                    \
    const int ka_ = (slab_) * sa_step, kw_ = (slab_) * sw_step;                                           \
    _Pragma("unroll") for (int i = 0; i < MT; ++i) n_a[i] =                                               \
        (unsigned)__builtin_amdgcn_raw_buffer_load_b32(rs_a, so_a[i], ka_, 0);                            \
    _Pragma("unroll") for (int j = 0; j < NT; ++j) n_w[j] = (unsigned)__builtin_amdgcn_raw_buffer_load_b32( \
        SWI && b_row[j] >= BN / 2 ? rs_w3 : rs_w, so_w[j], kw_, 0);                                       \
  } while (0)

  // fp8 fragment reads: each lane's byte offset inside a ring slot, for the
  // first row tile, per (k step, 16-byte half); the other row tiles sit a
  // multiple of 16 rows further (same swizzle), i.e. at an immediate offset
  int fa_off[F8 ? 2 * KS : 1], fb_off[F8 ? 2 * KS : 1];
  if constexpr (F8) {
#pragma unroll
    for (int q = 0; q < 2 * KS; ++q) {
      const int c = (q >> 1) * 4 + (q & 1) * 2 + hl;
      fa_off[q] = a_row[0] * RROW + ((c ^ swz(a_row[0])) << 4);
      fb_off[q] = b_row[0] * RROW + ((c ^ swz(b_row[0])) << 4);
    }
  }

  int a_issued = 0, consumed = 0;
  A_SETUP(at);
  B_SETUP(bt);
  // the first tile's first scales go out before its first slabs, so that
  // on every path the scale loads are followed by at least LDA A parts
  if constexpr (F8) {
    SC_SETUP(t_first);
    SC_LOAD(0);
  }
  ISSUE_A();
  ISSUE_B();
  ISSUE_A();
  int ca = 0, cb = 0;                           // ring positions of the slab being computed

  for (int ct = t_first; ct < t_end; ct += nslot) {
    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

    for (int kt = 0; kt < KT; ++kt) {
      // fp8: the A parts are issued every slab (into a dead ring slot once
      // the stream has ended), so the newest LDA loads are always A parts
      if (F8 || a_issued > consumed + 1) wait_vm<LDA>();
      else wait_vm<0>();
      if constexpr (F8) {
        // this slab's scales, loaded during the previous slab (raw dwords;
        // lanes of the upper half take blocks 1 and 3: shift them down)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          s_a[i] = n_a[i] >> (8 * hl);
          asm volatile("" : "+v"(s_a[i]));   // here, while the wait above covers the load
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          s_w[j] = n_w[j] >> (8 * hl);
          asm volatile("" : "+v"(s_w[j]));
        }
      }
      // Barrier without a memory fence: the wait covers this wave's slab
      // loads, and every wave is done with the slots about to be refilled.
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();

      // This iteration's loads, spread over the k steps with all W parts
      // before any A part (which keeps "only A(k + 1) follows W(k)" true).
      const bool do_b = bt < t_end, do_a = at < t_end;
      const char *sa = a_ring + ca * A_UNIT;
      const char *sb = b_ring + cb * B_UNIT;
      if constexpr (F8) {
        // k step ks covers k 64 ks .. 64 ks + 63 of the slab; lane half hl
        // supplies the 16-byte chunks 4 ks + hl and 4 ks + 2 + hl of its row
        // (the MFMA's k order: bytes j of lane l are k = 32 (j / 16) +
        // 16 (l / 32) + j % 16), and byte 2 ks of its scale dword is the
        // scale of block 2 ks + hl.  Fragments are read one A row tile
        // ahead and the next step's W tiles one step ahead; the empty asm
        // after each MFMA keeps it in place (otherwise the MFMAs drift
        // below the load bookkeeping and every fragment of the slab is
        // live at once, which spills the 256-row tile).
        typedef int i32x8 __attribute__((ext_vector_type(8)));
        i32x8 fa8[2], fb8[2][NT];
// fragment of the row tile drow_ rows past the first one (a multiple of 16)
#define F8_FRAG(dst_, base_, off_, drow_, ks_)                                                             \
  do {                                                                                                     \
    const u32x4 lo_ = *(const u32x4 *)((base_) + (off_)[2 * (ks_)] + (drow_) * RROW);                      \
    const u32x4 hi_ = *(const u32x4 *)((base_) + (off_)[2 * (ks_) + 1] + (drow_) * RROW);                  \
    dst_ = i32x8{(int)lo_[0], (int)lo_[1], (int)lo_[2], (int)lo_[3], (int)hi_[0], (int)hi_[1], (int)hi_[2], \
                 (int)hi_[3]};                                                                             \
  } while (0)
        // b_row[j] - b_row[0] and a_row[i] - a_row[0], compile-time
#define F8_BD(j_) (SWI ? ((j_) < H ? (j_) * 32 : BN / 2 + ((j_) - H) * 32) : (j_) * 32)
#define F8_AD(i_) ((i_) * 32)
#pragma unroll
        for (int j = 0; j < NT; ++j) F8_FRAG(fb8[0][j], sb, fb_off, F8_BD(j), 0);
        F8_FRAG(fa8[0], sa, fa_off, F8_AD(0), 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int cur = ks & 1;
          if (ks < KS / 2) {
            if (do_b) {
#pragma unroll
              for (int i = ks * PB; i < (ks + 1) * PB; ++i) ISSUE_B_PART(i);
            }
            // the next slab's scales (the next tile's first ones after the
            // last slab; the last slab of the last tile reloads its own):
            // after this slab's W parts and before its A parts, so the wait
            // at the top of the next slab, which leaves only the newest A
            // parts in flight, covers them a slab after they were issued
            if (ks == 0) {
              if (kt + 1 < KT) {
                SC_LOAD(kt + 1);
              } else if (ct + nslot < t_end) {
                SC_SETUP(ct + nslot);
                SC_LOAD(0);
              } else {
                SC_LOAD(kt);
              }
            }
          } else {
            // unconditional: once the A stream has ended (do_a false) these
            // refill the slot of the next, nonexistent slab from the last
            // tile's rows, which keeps the scale loads above followed by LDA
            // loads on every path (the wait at the top of the next slab then
            // leaves the A parts in flight without a compiler-inserted
            // vmcnt(0) for the scales)
#pragma unroll
            for (int i = (ks - KS / 2) * PA; i < (ks - KS / 2 + 1) * PA; ++i) ISSUE_A_PART(i);
          }
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            if (i + 1 < MT) F8_FRAG(fa8[(i + 1) & 1], sa, fa_off, F8_AD(i + 1), ks);
            else if (ks + 1 < KS) F8_FRAG(fa8[0], sa, fa_off, F8_AD(0), ks + 1);
            if (i == 0 && ks + 1 < KS) {
#pragma unroll
              for (int j = 0; j < NT; ++j) F8_FRAG(fb8[cur ^ 1][j], sb, fb_off, F8_BD(j), ks + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              if (ks == 0)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[cur][j], fa8[i & 1], acc[i][j], 0, 0,
                                                                            0, (int)s_w[j], 0, (int)s_a[i]);
              else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[cur][j], fa8[i & 1], acc[i][j], 0, 0,
                                                                            2, (int)s_w[j], 2, (int)s_a[i]);
              asm volatile("" : "+v"(acc[i][j]));
            }
          }
        }
#undef F8_FRAG
#undef F8_BD
#undef F8_AD
      } else {
      bf16x8 fa[2][MT], fb[2][NT];
#define READ_FRAGS(buf_, ks_)                                                                              \
  do {                                                                                                     \
    const int c_ = (ks_) * 2 + hl;                                                                         \
    _Pragma("unroll") for (int i = 0; i < MT; ++i) fa[buf_][i] =                                          \
        *(const bf16x8 *)(sa + a_row[i] * RROW + ((c_ ^ swz(a_row[i])) << 4));                            \
    _Pragma("unroll") for (int j = 0; j < NT; ++j) fb[buf_][j] =                                          \
        *(const bf16x8 *)(sb + b_row[j] * RROW + ((c_ ^ swz(b_row[j])) << 4));                            \
  } while (0)
      READ_FRAGS(0, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < KS) READ_FRAGS(cur ^ 1, ks + 1);
        if (ks < KS / 2) {
          if (do_b) {
#pragma unroll
            for (int i = ks * PB; i < (ks + 1) * PB; ++i) ISSUE_B_PART(i);
          }
        } else {
          if (do_a) {
#pragma unroll
            for (int i = (ks - KS / 2) * PA; i < (ks - KS / 2 + 1) * PA; ++i) ISSUE_A_PART(i);
          }
        }
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
      }
#undef READ_FRAGS
      }
      if (do_b) STEP_B();
      if (do_a) STEP_A();
      ca = ca + 1 == NA ? 0 : ca + 1;
      cb = cb + 1 == NB ? 0 : cb + 1;
      ++consumed;
    }

    store_tile<EPI, MT, NT, WTM, WTN>(acc, p0, p1, qo, ct, tiles0, ntm0, ntm1, ntn, GM, BM, OUTC, wm, wn, lane);
  }
  // fp8 leaves its last refills of dead ring slots in flight: they land
  // before the workgroup's LDS is released
  if constexpr (F8) wait_vm<0>();
#undef SC_SETUP
#undef SC_LOAD
#undef ISSUE_A
#undef ISSUE_B
#undef ISSUE_A_PART
#undef ISSUE_B_PART
#undef STEP_A
#undef STEP_B
#undef A_SETUP
#undef B_SETUP
}

// ------------------------------------------------------------ ping-pong
// 256 x 256 tiles with 8 waves in two groups of four (waves 0-3 and 4-7; the
// dispatcher puts waves w and w + 4 on one SIMD, so every SIMD holds one
// wave of each group).  Group g owns tile rows 128 g .. 128 g + 127 (its own
// half of the A panel) and wave j of a group the 64 output columns from 64 j
// (SwiGLU: 32 columns of w1 and the same 32 of w3), 128 x 64 per wave as in
// gemm_bf16.  A wave handles each 64-deep slab in two phases: a memory phase
// that issues its share of the global loads and reads all of its fragments
// of the slab from LDS into registers, then a compute phase of 32 MFMAs on
// them.  The groups run one phase apart with a workgroup barrier between
// phases, so on every SIMD one wave issues MFMAs from registers while the
// other reads LDS and issues loads: the matrix core does not wait for a
// barrier, for the first fragments of a slab or for the issue of loads (a
// direct-to-LDS load instruction holds its wave for tens of cycles, so no
// load is issued from a compute phase).
//
// LDS (160 KB): A in two stages [A0 | A1], W in three stages [W0 | W1 | W2],
// 32 KB each (256 rows x 128 bytes; chunk c of row r in slot
// c ^ ((r >> 1) & 7), as in gemm_bf16).  Slab s uses A stage s & 1 and W
// stage s % 3.  Group g reads its A rows of slab s in its memory phase of s
// (phase 2s + g) and both groups read all W rows of s, so:
//  * each group loads its own 128 A rows of slab s + 1 in its memory phase
//    of slab s (that half of the stage was last read by the same group in
//    phase 2s + g - 2), waited for at the end of its next compute phase;
//  * group 0 loads W rows 0-127 of slab s + 1 and group 1 W rows 128-255 of
//    slab s + 2 in their memory phases of s (the W stage of slab s + 2 last
//    held slab s - 1, read by phase 2s - 1); group 1 waits for its W half
//    at the end of its memory phase of s + 1, before the barrier that opens
//    group 0's reads of slab s + 2.
// Rows past the end of A read as zeros through the buffer bounds (their
// outputs are not stored).  A finished tile's epilogue runs in the wave's
// next memory phase, while the other group computes.
template <int EPI, int GM>
__global__ __launch_bounds__(512) void gemm_pp(GemmProblem p0, GemmProblem p1, int tiles0, int ntm0, int ntm1,
                                               int total_tiles, int per_xcd, QkvOut qo) {
  using namespace gk;
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr int KS = RBK / 16;
  constexpr bool SWI = (EPI == EPI_SWIGLU);
  constexpr int OUTC = SWI ? BN / 2 : BN;
  constexpr int H = SWI ? NT / 2 : NT;
  constexpr int UNIT = BM * RROW;               // one stage of A or W: 32 KB
  constexpr int W_BASE = 2 * UNIT;
  static_assert(BM == BN && UNIT == 32768, "A stage select is address bit 15");
  static_assert(EPI != EPI_QKV || WTN == 64, "QKV epilogue: one head per wave");
  __shared__ __attribute__((aligned(1024))) char smem[5 * UNIT];

  const int xcd = blockIdx.x & 7, nslot = gridDim.x >> 3;
  const int t_end = min((xcd + 1) * per_xcd, total_tiles);
  const int t_first = xcd * per_xcd + (blockIdx.x >> 3);
  if (t_first >= t_end) return;
  const int n_tiles = (t_end - t_first + nslot - 1) / nslot;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wj = wave & 3;
  const int wm = grp, wn = wj;
  const int ntn = p0.N / OUTC;
  const int K = p0.K, KT = K / RBK;
  const int n_slabs = n_tiles * KT;
  const int lrow = lane >> 3, lslot = lane & 7;
  const int frow = lane & 31, hl = lane >> 5;

  // ---- this wave's loads: rows 128 grp + 32 i + 8 wj + lrow (i < 4) of the
  // A panel and of the W panel, 8 rows x 128 bytes per instruction; one
  // per-lane offset per operand (32 i rows ride in the scalar offset)
  const int hrow = grp * 128 + wj * 8;          // first row of instruction 0 (uniform)
  const int lsw = (lslot ^ swz(hrow + lrow)) * 16;
  const int rstride = 32 * K * 2;
  int a_off = 0, b_off = 0;
  __amdgpu_buffer_rsrc_t rs_a, rs_w;
  int at = t_first, akt = 0, bt = t_first, bkt = 0;   // next slab of the A / W streams
  int a_slab = 0;                                     // its index in this workgroup's slab order
#define PP_SETUP_A(t_)                                                                                   \
  do {                                                                                                   \
    bool sec_;                                                                                           \
    int m0_, n0_;                                                                                        \
    tile_coords(t_, tiles0, ntm0, ntm1, ntn, GM, BM, OUTC, sec_, m0_, n0_);                              \
    const int ab_ = __builtin_amdgcn_readfirstlane((sec_ ? p1.M : p0.M) * K * 2);                        \
    a_off = (int)__umul24(m0_ + hrow + lrow, K * 2) + lsw;                                               \
    rs_a = __builtin_amdgcn_make_buffer_rsrc((void *)(sec_ ? p1.A : p0.A), (short)0, ab_, 0x00020000);   \
  } while (0)
#define PP_SETUP_W(t_)                                                                                   \
  do {                                                                                                   \
    bool sec_;                                                                                           \
    int m0_, n0_;                                                                                        \
    tile_coords(t_, tiles0, ntm0, ntm1, ntn, GM, BM, OUTC, sec_, m0_, n0_);                              \
    const void *wp_ = (SWI && grp == 1) ? (sec_ ? p1.W3 : p0.W3) : (sec_ ? p1.W : p0.W);                  \
    b_off = (int)__umul24(n0_ + (SWI ? hrow - grp * 128 : hrow) + lrow, K * 2) + lsw;                     \
    rs_w = __builtin_amdgcn_make_buffer_rsrc((void *)wp_, (short)0, p0.N * K * 2, 0x00020000);            \
  } while (0)
#define PP_LOAD_A()                                                                                      \
  do {                                                                                                   \
    char *d_ = smem + (a_slab & 1) * UNIT + hrow * RROW;                                                 \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) __builtin_amdgcn_raw_ptr_buffer_load_lds(               \
        rs_a, (lds_void *)(d_ + i * 32 * RROW), 16, a_off, akt * RROW + i * rstride, 0, 0);              \
    ++a_slab;                                                                                            \
    if (++akt == KT) {                                                                                   \
      akt = 0;                                                                                           \
      at += nslot;                                                                                       \
      if (at < t_end) PP_SETUP_A(at);                                                                    \
    }                                                                                                    \
  } while (0)
#define PP_LOAD_W(st_)                                                                                   \
  do {                                                                                                   \
    char *d_ = smem + W_BASE + (st_) * UNIT + hrow * RROW;                                               \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) __builtin_amdgcn_raw_ptr_buffer_load_lds(               \
        rs_w, (lds_void *)(d_ + i * 32 * RROW), 16, b_off, bkt * RROW + i * rstride, 0, 0);              \
    if (++bkt == KT) {                                                                                   \
      bkt = 0;                                                                                           \
      bt += nslot;                                                                                       \
      if (bt < t_end) PP_SETUP_W(bt);                                                                    \
    }                                                                                                    \
  } while (0)

  // ---- fragments.  Row tile i of this wave's A rows is wm * 128 + 32 i +
  // frow, W row tile j is b_row0 + bd(j); the swizzle of all of them is that
  // of frow, so one address per k step and operand, tiles at immediate
  // offsets.  A stage = address bit 15; the W stage moves by 32 KB a slab.
  const int sf = swz(frow);
  const int b_row0 = (SWI ? wn * (WTN / 2) : wn * WTN) + frow;
  int a_addr[KS], w_addr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int ch = ((ks * 2 + hl) ^ sf) << 4;
    a_addr[ks] = (wm * WTM + frow) * RROW + ch;
    w_addr[ks] = W_BASE + b_row0 * RROW + ch;
  }
  bf16x8 fa[KS][MT], fb[KS][NT];
#define PP_BD(j_) ((SWI ? ((j_) < H ? (j_) * 32 : BN / 2 + ((j_) - H) * 32) : (j_) * 32) * RROW)
#define PP_READ()                                                                                        \
  do {                                                                                                   \
    _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                                  \
      _Pragma("unroll") for (int i = 0; i < MT; ++i) fa[ks][i] =                                         \
          *(const bf16x8 *)(smem + a_addr[ks] + i * 32 * RROW);                                          \
      _Pragma("unroll") for (int j = 0; j < NT; ++j) fb[ks][j] = *(const bf16x8 *)(smem + w_addr[ks] + PP_BD(j)); \
    }                                                                                                    \
  } while (0)
#define PP_BARRIER()                                                                                     \
  do {                                                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                                   \
    __builtin_amdgcn_s_barrier();                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                                   \
  } while (0)

  f32x16 acc[MT][NT];
  int ct = t_first, ckt = 0;   // tile and slab being computed
  int wst = 0;                 // W stage of slab s
  // ---- prologue: slab 0 from every wave (its A rows and its W half), and
  // group 1's W half of slab 1
  PP_SETUP_A(t_first);
  PP_SETUP_W(t_first);
  PP_LOAD_A();
  PP_LOAD_W(0);
  const bool w1_ahead = grp == 1 && n_slabs > 1;
  if (w1_ahead) PP_LOAD_W(1);
  if (w1_ahead) wait_vm<4>();
  else wait_vm<0>();
  PP_BARRIER();
  if (grp == 1) PP_BARRIER();   // group 1 runs one phase behind

  for (int s = 0;; ++s) {
    // ---- memory phase of slab s: this wave's loads for later slabs, the
    // finished tile's epilogue, then the fragments of slab s
    const int w1 = wst == 2 ? 0 : wst + 1, w2 = w1 == 2 ? 0 : w1 + 1;
    const bool la = s + 1 < n_slabs;                       // A rows of slab s + 1
    const bool lw = grp == 0 ? s + 1 < n_slabs : s + 2 < n_slabs;   // W half of slab s + 1 / s + 2
    if (la) PP_LOAD_A();
    if (lw) PP_LOAD_W(grp == 0 ? w1 : w2);
    const bool epi = ckt == 0 && s > 0;
    if (epi)
      store_tile<EPI, MT, NT, WTM, WTN>(acc, p0, p1, qo, ct - nslot, tiles0, ntm0, ntm1, ntn, GM, BM, OUTC, wm, wn,
                                        lane);
    if (s == n_slabs) break;
    __builtin_amdgcn_sched_barrier(0);
    PP_READ();
    wait_lgkm0();
    // group 1: its W half of slab s + 1 (issued a slab ago) has landed; this
    // phase's loads stay in flight (an epilogue's stores make it wait for all)
    if (grp == 1) {
      if (epi) wait_vm<0>();
      else if (la && lw) wait_vm<8>();
      else if (la || lw) wait_vm<4>();
      else wait_vm<0>();
    }
    PP_BARRIER();
    // ---- compute phase of slab s (a tile's first k step starts its
    // accumulators from zero in the MFMA itself, not from 128 moves)
    if (ckt == 0) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][j], fa[0][i], f32x16{}, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][j], fa[0][i], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int ks = 1; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
    if (++ckt == KT) {
      ckt = 0;
      ct += nslot;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      a_addr[ks] ^= UNIT;
      w_addr[ks] += wst == 2 ? -2 * UNIT : UNIT;
    }
    wst = w1;
    // this wave's A rows of slab s + 1 have landed (group 1 leaves its W half
    // of slab s + 2, issued after them, in flight)
    if (grp == 1 && lw && !epi) wait_vm<4>();
    else wait_vm<0>();
    PP_BARRIER();
  }
  if (grp == 0) PP_BARRIER();   // pairs with group 1's barrier after its last compute phase
#undef PP_BD
#undef PP_BARRIER
#undef PP_READ
#undef PP_LOAD_A
#undef PP_LOAD_W
#undef PP_SETUP_A
#undef PP_SETUP_W
}

// LENS_GEMM_PP=0 in the environment keeps the SwiGLU and gated residual
// projections on gemm_bf16 (for side-by-side measurement); read once.
bool lens_gemm_pp_off() {
  static const bool off = [] {
    const char *e = getenv("LENS_GEMM_PP");
    return e && e[0] == '0';
  }();
  return off;
}

// Persistent launch: at most one workgroup per CU, a multiple of 8 so that
// every XCD gets the same number of workgroups.
// GEMM kernels launched by the current thread's last launch_gemm /
// launch_gemm_fp8 call (a call may split into two launches).
thread_local int g_gemm_kernels = 0;

int cu_count() {
  static int n[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 256;
  if (n[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    n[dev] = c;
  }
  return n[dev];
}

// Both problems of a grouped launch must share N and K (the image and text
// weights of one layer do); N must be a multiple of the tile's output
// columns and K of the slab depth.
template <int BM, int BN, int WM, int WN, int EPI, int GM = 4, bool BUF = false, bool F8 = false>
hipError_t run_bf16(const GemmProblem *pr, int np, hipStream_t st, const QkvOut *qo = nullptr, int max_grid = 0) {
  constexpr bool SWI = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX);
  const int outc = SWI ? BN / 2 : BN;
  if (np > 1 && (pr[0].N != pr[1].N || pr[0].K != pr[1].K)) return hipErrorInvalidValue;
  if (pr[0].N % outc || pr[0].K % (F8 ? 128 : gk::RBK) || pr[0].K <= 0) return hipErrorInvalidValue;
  if constexpr (F8) {
    for (int i = 0; i < np; ++i)
      if (pr[i].M > 0 && (!pr[i].A_scale || !pr[i].W_scale || (SWI && !pr[i].W3_scale) ||
                          (EPI == EPI_SWIGLU_MX && !pr[i].C_scale)))
        return hipErrorInvalidValue;
  }
  int ntm[2] = {0, 0}, tiles[2] = {0, 0};
  for (int i = 0; i < np; ++i) {
    ntm[i] = (pr[i].M + BM - 1) / BM;
    tiles[i] = pr[i].M > 0 ? ntm[i] * (pr[i].N / outc) : 0;
  }
  const int total = tiles[0] + tiles[1];
  if (total == 0) return hipSuccess;
  const int per_xcd = (total + 7) / 8;
  int grid = (max_grid > 0 ? max_grid : cu_count()) / 8 * 8;
  if (grid > per_xcd * 8) grid = per_xcd * 8;
  GemmProblem q0 = pr[0], q1 = np > 1 ? pr[1] : pr[0];
  if (tiles[0] == 0) q0 = q1;
  QkvOut qv = {};
  if constexpr (EPI == EPI_QKV) {
    if (!qo) return hipErrorInvalidValue;
    qv = *qo;
  }
  ++g_gemm_kernels;
  hipLaunchKernelGGL((gemm_bf16<BM, BN, WM, WN, EPI, GM, BUF, F8>), dim3(grid), dim3(64 * WM * WN), 0, st, q0, q1, tiles[0],
                     ntm[0] > 0 ? ntm[0] : 1, ntm[1] > 0 ? ntm[1] : 1, total, per_xcd, qv);
  return hipGetLastError();
}

// Launch of the ping-pong kernel (256 x 256 tiles, buffer loads: every
// operand below 2 GiB); grouping and XCD mapping as run_bf16.
template <int EPI, int GM = 4>
hipError_t run_pp(const GemmProblem *pr, int np, hipStream_t st, const QkvOut *qo = nullptr, int max_grid = 0) {
  constexpr bool SWI = EPI == EPI_SWIGLU;
  const int outc = SWI ? 128 : 256;
  if (np > 1 && (pr[0].N != pr[1].N || pr[0].K != pr[1].K)) return hipErrorInvalidValue;
  if (pr[0].N % outc || pr[0].K % gk::RBK || pr[0].K <= 0) return hipErrorInvalidValue;
  int ntm[2] = {0, 0}, tiles[2] = {0, 0};
  for (int i = 0; i < np; ++i) {
    ntm[i] = (pr[i].M + 255) / 256;
    tiles[i] = pr[i].M > 0 ? ntm[i] * (pr[i].N / outc) : 0;
  }
  const int total = tiles[0] + tiles[1];
  if (total == 0) return hipSuccess;
  const int per_xcd = (total + 7) / 8;
  int grid = (max_grid > 0 ? max_grid : cu_count()) / 8 * 8;
  if (grid > per_xcd * 8) grid = per_xcd * 8;
  GemmProblem q0 = pr[0], q1 = np > 1 ? pr[1] : pr[0];
  if (tiles[0] == 0) q0 = q1;
  QkvOut qv = {};
  if constexpr (EPI == EPI_QKV) {
    if (!qo) return hipErrorInvalidValue;
    qv = *qo;
  }
  ++g_gemm_kernels;
  hipLaunchKernelGGL((gemm_pp<EPI, GM>), dim3(grid), dim3(512), 0, st, q0, q1, tiles[0], ntm[0] > 0 ? ntm[0] : 1,
                     ntm[1] > 0 ? ntm[1] : 1, total, per_xcd, qv);
  return hipGetLastError();
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
  ++g_gemm_kernels;
  hipLaunchKernelGGL((gemm_f32_simple<EPI>), dim3(total), dim3(256), 0, st, pr[0], q1, tiles[0], ntm[0], ntm[1]);
  return hipGetLastError();
}

}  // namespace

// bf16 tile choice: 256 x 256 tiles, or 128 x 256 when those would leave
// most CUs idle, or 256 x 128 when N is not a multiple of 256 (N = 128
// for the final projection).
// Whether a grouped launch of two problems (image rows, text rows) runs
// faster as the first problem alone in 256 x 256 tiles, then the second in
// 128 x 256 tiles: rounds of full tiles on the CUs + 0.68 x rounds of half
// tiles (a half tile takes ~0.68 of a full one) against the grouped
// launch's rounds.
static bool split_second_problem(const GemmProblem *pr, int np, int outc) {
  if (np != 2 || pr[0].M <= 0 || pr[1].M <= 0) return false;
  const int C = cu_count();
  const int t0 = ((pr[0].M + 255) / 256) * (pr[0].N / outc);
  const int t1 = ((pr[1].M + 255) / 256) * (pr[1].N / outc);
  const int h1 = ((pr[1].M + 127) / 128) * (pr[1].N / outc);
  const double grouped = (double)((t0 + t1 + C - 1) / C);
  const double split = (double)((t0 + C - 1) / C) + 0.68 * (double)((h1 + C - 1) / C);
  return split + 0.2 < grouped;
}

template <int EPI>
hipError_t dispatch_bf16(const GemmProblem *pr, int np, hipStream_t st, const QkvOut *qo) {
  constexpr bool SWI = EPI == EPI_SWIGLU;
  const int outc = SWI ? 128 : 256;   // output columns of a 256-wide tile
  bool n256 = true;
  int tiles256 = 0;
  for (int i = 0; i < np; ++i) {
    if (pr[i].N % outc) n256 = false;
    tiles256 += ((pr[i].M + 255) / 256) * (pr[i].N / outc);
  }
  // buffer loads (32-bit offsets) whenever every operand spans < 2 GiB
  bool buf = true;
  for (int i = 0; i < np; ++i)
    if ((int64_t)pr[i].M * pr[i].K * 2 >= (int64_t(1) << 31) || (int64_t)pr[i].N * pr[i].K * 2 >= (int64_t(1) << 31))
      buf = false;
  if (!n256) {
    if constexpr (SWI || EPI == EPI_QKV) return hipErrorInvalidValue;
    else return buf ? run_bf16<256, 128, 4, 2, EPI, 4, true>(pr, np, st, qo) : run_bf16<256, 128, 4, 2, EPI>(pr, np, st, qo);
  }
  if (tiles256 * 2 < cu_count())
    return buf ? run_bf16<128, 256, 2, 4, EPI, 4, true>(pr, np, st, qo) : run_bf16<128, 256, 2, 4, EPI>(pr, np, st, qo);
  // w1 | w3 with the SwiGLU epilogue: the ping-pong kernel (1.09-1.15x the
  // gemm_bf16 loop at the 1024^2 CFG shape)
  if constexpr (SWI) {
    if (buf && !lens_gemm_pp_off()) {
      // A grouped (image, text) launch whose text tiles spill into a partial
      // last round: the image problem alone in 256 x 256 tiles, then the
      // text problem in 128 x 256 tiles, when the rounds that costs (a half
      // tile takes ~0.68 of a full one) beat the grouped launch's.  At the
      // 1024^2 CFG shape: 1024 image tiles (4 rounds on 256 CUs) + 128 text
      // tiles (a fifth, half-empty round) become 4 rounds + one round of
      // 256 half tiles.
      if (split_second_problem(pr, np, outc)) {
        const hipError_t e = run_pp<EPI>(pr, 1, st, qo);
        if (e != hipSuccess) return e;
        return run_bf16<128, 256, 2, 4, EPI, 4, true>(pr + 1, 1, st, qo);
      }
      return run_pp<EPI>(pr, np, st, qo);
    }
  }
  // the gated residual GEMMs (out-proj, w2) also run on the ping-pong loop
  // (measured 0.9 % faster per GEMM launch on the step; QKV stays on
  // gemm_bf16, 0.5 % slower there)
  if constexpr (EPI == EPI_GATED) {
    if (buf && !lens_gemm_pp_off()) return run_pp<EPI>(pr, np, st, qo);
  }
  return buf ? run_bf16<256, 256, 2, 4, EPI, 4, true>(pr, np, st, qo) : run_bf16<256, 256, 2, 4, EPI>(pr, np, st, qo);
}

// fp8: the bf16 tile choice (256 x 256, or 128 x 256 when 256-row tiles
// would leave most CUs idle); every operand must be below 2 GiB (buffer
// loads)
template <int EPI>
hipError_t dispatch_fp8(const GemmProblem *pr, int np, hipStream_t st, const QkvOut *qo) {
  constexpr bool SWI = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX;
  const int outc = SWI ? 128 : 256;
  int tiles256 = 0;
  for (int i = 0; i < np; ++i) {
    if (pr[i].N % outc) return hipErrorInvalidValue;
    if ((int64_t)pr[i].M * pr[i].K >= (int64_t(1) << 31) || (int64_t)pr[i].N * pr[i].K >= (int64_t(1) << 31))
      return hipErrorInvalidValue;
    tiles256 += ((pr[i].M + 255) / 256) * (pr[i].N / outc);
  }
  // (the text rows of w1 | w3 in a separate round of half tiles, as on the
  // bf16 path, measured no faster here: fp8 GEMMs 17.51 against 17.57 ms
  // per step, within the step's noise)
  if (tiles256 * 2 < cu_count()) return run_bf16<128, 256, 2, 4, EPI, 4, true, true>(pr, np, st, qo);
  return run_bf16<256, 256, 2, 4, EPI, 4, true, true>(pr, np, st, qo);
}

hipError_t launch_gemm_fp8(int epi, const GemmProblem *probs, int nprob, hipStream_t stream, const QkvOut *qo) {
  g_gemm_kernels = 0;
  switch (epi) {
    case EPI_STORE: return dispatch_fp8<EPI_STORE>(probs, nprob, stream, nullptr);
    case EPI_GATED: return dispatch_fp8<EPI_GATED>(probs, nprob, stream, nullptr);
    case EPI_SWIGLU: return dispatch_fp8<EPI_SWIGLU>(probs, nprob, stream, nullptr);
    case EPI_SWIGLU_MX: return dispatch_fp8<EPI_SWIGLU_MX>(probs, nprob, stream, nullptr);
    case EPI_QKV: return dispatch_fp8<EPI_QKV>(probs, nprob, stream, qo);
  }
  return hipErrorInvalidValue;
}

int gemm_kernels_launched() { return g_gemm_kernels; }

hipError_t launch_gemm(int epi, bool bf16_path, const GemmProblem *probs, int nprob, hipStream_t stream,
                       const QkvOut *qo) {
  g_gemm_kernels = 0;
  if (bf16_path) {
    switch (epi) {
      case EPI_STORE: return dispatch_bf16<EPI_STORE>(probs, nprob, stream, nullptr);
      case EPI_STORE_F32: return dispatch_bf16<EPI_STORE_F32>(probs, nprob, stream, nullptr);
      case EPI_GATED: return dispatch_bf16<EPI_GATED>(probs, nprob, stream, nullptr);
      case EPI_SWIGLU: return dispatch_bf16<EPI_SWIGLU>(probs, nprob, stream, nullptr);
      case EPI_QKV: return dispatch_bf16<EPI_QKV>(probs, nprob, stream, qo);
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

namespace lens {
// ping-pong launchers, selectable for measurement
hipError_t launch_gemm_pp(int epi, const GemmProblem *probs, int nprob, hipStream_t stream, const QkvOut *qo) {
  switch (epi) {
    case EPI_STORE: return run_pp<EPI_STORE>(probs, nprob, stream, nullptr);
    case EPI_STORE_F32: return run_pp<EPI_STORE_F32>(probs, nprob, stream, nullptr);
    case EPI_GATED: return run_pp<EPI_GATED>(probs, nprob, stream, nullptr);
    case EPI_SWIGLU: return run_pp<EPI_SWIGLU>(probs, nprob, stream, nullptr);
    case EPI_QKV: return run_pp<EPI_QKV>(probs, nprob, stream, qo);
  }
  return hipErrorInvalidValue;
}
}  // namespace lens

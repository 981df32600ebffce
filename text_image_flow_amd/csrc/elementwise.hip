// Bandwidth-bound kernels of the denoiser step:
//   * RMSNorm + AdaLN modulation (Lens-Turbo-3.8B-bf16 article, "自适应调制与
//     RMSNorm"; shift/scale/gate order from the Lens blog's "Overview");
//   * per-head QK RMSNorm + 3-axis RoPE, writing the joint attention layout
//     (same article: norm_q/norm_k/norm_added_q/norm_added_k; "3D RoPE",
//     axes [8, 28, 28]);
//   * the skinny GEMM of AdaLN and the timestep MLP (time_text_embed);
//   * timestep sinusoid; per-layer text-feature RMSNorm (txt_norm.0..3);
//   * the CFG + Euler flow step (SOTA image-generation survey, "CFG" and
//     "Rectified Flow"; the flow-matching path of the Lens paper summary),
//     plain or with the norm-rescaled combine (Lens blog, "Exploring Image
//     Editing");
//   * MX fp8 quantization (Lens-3.8B-4bit article, section 4), also fused
//     into norm+modulate as an output format.
// Statistics and arithmetic are float32; stores round to the storage type.
#include "common.h"

namespace lens {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T>
__device__ __forceinline__ void store4(T *dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float *dst, float a, float b, float c, float d) {
  *(float4 *)dst = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16 *dst, float a, float b, float c, float d) {
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *(bf16x4 *)dst = v;
}

// ------------------------------------------------ RMSNorm + modulation
// norm_rw(MX) rows per wave; D % 256 == 0 so each lane owns D/256 float4
// groups of a row.  Three rows per wave for bf16 / fp32 output, four for MX
// fp8 output.  The normalized rows are stored non-temporally (they are read
// once, by the next GEMM, long after this kernel's other traffic).  Measured
// on MI355X at 1024^2 (9216 rows of 1536, h just written by the previous
// GEMM): 3 rows + non-temporal stores 14.1 us, 2 rows + ordinary stores
// 15.5 us; non-temporal loads of h are slower there (h is still in cache).
constexpr int norm_rw(bool mx) { return mx ? 4 : 3; }

template <typename T>
__device__ __forceinline__ void store4_nt(T *dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4_nt<float>(float *dst, float a, float b, float c, float d) {
  __builtin_nontemporal_store(f32x4{a, b, c, d}, (f32x4 *)dst);
}
template <>
__device__ __forceinline__ void store4_nt<bf16>(bf16 *dst, float a, float b, float c, float d) {
  __builtin_nontemporal_store(bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d}, (bf16x4 *)dst);
}

template <typename T, int G, bool MX = false>
__global__ __launch_bounds__(256) void norm_modulate_kernel(NormModProblem p0, NormModProblem p1, int split0,
                                                            float eps) {
  constexpr int D = G * 256;
  constexpr int NORM_RW = norm_rw(MX);
  // NORM_RW consecutive rows per wave (problem 0's row count is padded to
  // split0 so that no wave straddles the two problems); the sample's shift
  // and scale stay in registers, and the next row's loads go out before this
  // row's reduction.
  int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * NORM_RW;
  const int lane = threadIdx.x & 63;
  const bool second = row >= split0;
  const NormModProblem p = second ? p1 : p0;
  if (second) row -= split0;
  const int rows = p.rows;
  if (row >= rows) return;
  int cur_b = -1;
  float4 s4[G], h4[G], v[G];
#pragma unroll
  for (int i = 0; i < G; ++i) v[i] = *(const float4 *)(p.h + (int64_t)row * D + (i * 64 + lane) * 4);
  for (int rr = 0; rr < NORM_RW; ++rr) {
    const int r = row + rr;
    if (r >= rows) break;
    const bool more = rr + 1 < NORM_RW && r + 1 < rows;
    float4 nv[G];
    if (more) {
#pragma unroll
      for (int i = 0; i < G; ++i) nv[i] = *(const float4 *)(p.h + (int64_t)(r + 1) * D + (i * 64 + lane) * 4);
    }
    const int b = r / p.rows_per_sample;
    if (b != cur_b) {
      cur_b = b;
      const float *sh = p.shift + (int64_t)b * p.mod_stride, *sc = p.scale + (int64_t)b * p.mod_stride;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        s4[i] = *(const float4 *)(sc + (i * 64 + lane) * 4);
        h4[i] = *(const float4 *)(sh + (i * 64 + lane) * 4);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    ss = wave_sum(ss);
    const float rs = rsqrtf(ss / (float)D + eps);
    if constexpr (MX) {
      // MX fp8 row: the 8 lanes of a 32-column block agree on its scale
      // through three xor exchanges, each lane packs its 4 columns
      unsigned *out = (unsigned *)((unsigned char *)p.out + (int64_t)r * D);
      unsigned char *osc = (unsigned char *)p.out_scale;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float y0 = v[i].x * rs * (1.f + s4[i].x) + h4[i].x, y1 = v[i].y * rs * (1.f + s4[i].y) + h4[i].y;
        const float y2 = v[i].z * rs * (1.f + s4[i].z) + h4[i].z, y3 = v[i].w * rs * (1.f + s4[i].w) + h4[i].w;
        float am = fmaxf(fmaxf(fabsf(y0), fabsf(y1)), fmaxf(fabsf(y2), fabsf(y3)));
        am = fmaxf(am, __shfl_xor(am, 1));
        am = fmaxf(am, __shfl_xor(am, 2));
        am = fmaxf(am, __shfl_xor(am, 4));
        const int ex = mx_exponent(am);
        out[i * 64 + lane] = mx_pack4(y0, y1, y2, y3, ex);
        if ((lane & 7) == 0) osc[mx_scale_index(r, (i * 64 + lane) >> 3, rows)] = (unsigned char)(ex + 127);
      }
    } else {
      T *out = (T *)p.out + (int64_t)r * D;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int c = (i * 64 + lane) * 4;
        store4_nt<T>(out + c, v[i].x * rs * (1.f + s4[i].x) + h4[i].x, v[i].y * rs * (1.f + s4[i].y) + h4[i].y,
                     v[i].z * rs * (1.f + s4[i].z) + h4[i].z, v[i].w * rs * (1.f + s4[i].w) + h4[i].w);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < G; ++i) v[i] = nv[i];
    }
  }
}

// ------------------------------------------------ QK RMSNorm + RoPE
// Block = 64 joint positions x one head; thread t: position t/4, dims
// [(t%4)*16, +16).  V is transposed through LDS so V^T rows are written as
// contiguous 128-byte runs.
template <typename T>
__device__ __forceinline__ void load16(const T *src, float *v) {
  for (int i = 0; i < 16; ++i) v[i] = to_f32(src[i]);
}
template <>
__device__ __forceinline__ void load16<bf16>(const bf16 *src, float *v) {
  const bf16x8 a = *(const bf16x8 *)src, b = *(const bf16x8 *)(src + 8);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = (float)a[i];
    v[8 + i] = (float)b[i];
  }
}
template <typename T>
__device__ __forceinline__ void store16(T *dst, const float *v) {
  for (int i = 0; i < 16; ++i) dst[i] = from_f32<T>(v[i]);
}
template <>
__device__ __forceinline__ void store16<bf16>(bf16 *dst, const float *v) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)v[i];
    b[i] = (bf16)v[8 + i];
  }
  *(bf16x8 *)dst = a;
  *(bf16x8 *)(dst + 8) = b;
}

template <typename T>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(QkRopeArgs a) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int t = threadIdx.x, tok = t >> 2, qd = t & 3, d0 = qd * 16;
  const int p = blockIdx.x * 64 + tok;
  const int S = a.S_img + a.S_txt;
  const int D = a.H * 64;
  const int64_t bh = (int64_t)b * a.H + h;
  T *Qo = (T *)a.Q + (bh * a.S_pad + p) * 64 + d0;
  T *Ko = (T *)a.K + (bh * a.S_pad + p) * 64 + d0;

  float q[16], k[16], v[16];
  bool live = p < S;
  const T *src = nullptr;
  const T *qg = nullptr, *kg = nullptr;
  const int32_t *pos = nullptr;
  if (p < a.S_img) {
    src = (const T *)a.qkv_img + ((int64_t)b * a.S_img + p) * 3 * D;
    qg = (const T *)a.qg_img;
    kg = (const T *)a.kg_img;
    pos = a.pos_img + 3 * p;
  } else if (live) {
    src = (const T *)a.qkv_txt + ((int64_t)b * a.S_txt + (p - a.S_img)) * 3 * D;
    qg = (const T *)a.qg_txt;
    kg = (const T *)a.kg_txt;
    pos = a.pos_txt + 3 * (p - a.S_img);
  }
  if (live) {
    load16<T>(src + h * 64 + d0, q);
    load16<T>(src + D + h * 64 + d0, k);
    load16<T>(src + 2 * D + h * 64 + d0, v);
  } else {
    for (int i = 0; i < 16; ++i) q[i] = k[i] = v[i] = 0.f;
  }
  float sq = 0.f, sk = 0.f;
  for (int i = 0; i < 16; ++i) {
    sq += q[i] * q[i];
    sk += k[i] * k[i];
  }
  // the four threads of a position are lanes 4j..4j+3 of one wave
  sq += __shfl_xor(sq, 1);
  sq += __shfl_xor(sq, 2);
  sk += __shfl_xor(sk, 1);
  sk += __shfl_xor(sk, 2);
  if (live) {
    const float rq = rsqrtf(sq / 64.f + a.eps), rk = rsqrtf(sk / 64.f + a.eps);
    const float p0 = (float)pos[0], p1 = (float)pos[1], p2 = (float)pos[2];
    const float l2t = log2f(a.theta);
    for (int i = 0; i < 16; i += 2) {
      const int d = d0 + i;
      // axis segment and pair index inside it
      float pa, j, w;
      if (d < a.axes0) {
        pa = p0; j = (float)(d / 2); w = (float)a.axes0;
      } else if (d < a.axes0 + a.axes1) {
        pa = p1; j = (float)((d - a.axes0) / 2); w = (float)a.axes1;
      } else {
        pa = p2; j = (float)((d - a.axes0 - a.axes1) / 2); w = (float)a.axes2;
      }
      const float ang = pa * exp2f(-2.f * j / w * l2t);
      float sn, cs;
      sincosf(ang, &sn, &cs);
      const float q0 = q[i] * rq * to_f32(qg[d]), q1 = q[i + 1] * rq * to_f32(qg[d + 1]);
      const float k0 = k[i] * rk * to_f32(kg[d]), k1 = k[i + 1] * rk * to_f32(kg[d + 1]);
      q[i] = (q0 * cs - q1 * sn) * a.q_scale;
      q[i + 1] = (q0 * sn + q1 * cs) * a.q_scale;
      k[i] = k0 * cs - k1 * sn;
      k[i + 1] = k0 * sn + k1 * cs;
    }
  }
  store16<T>(Qo, q);
  store16<T>(Ko, k);
  store16<T>((T *)a.V + (bh * a.S_pad + p) * 64 + d0, v);
}

// ------------------------------------------------ skinny GEMM (GEMV)
// y[b, n] = sum_k f(x[b, k]) W[n, k] + bias[n] for b < B (B <= 8 per launch).
// HBM-bound on W, which is read exactly once for all B samples.  (fp32 weights;
// bf16 weights use gemv_bf16_kernel below.)  Each wave
// keeps f(x) for its k-range in registers (lane l owns k = 8 l + 512 i) and
// handles 8 rows at a time with all of their 16-byte weight loads issued
// before any FMA, so many loads are in flight per lane.
constexpr int GEMV_ROWS = 8;      // rows per wave pass
constexpr int GEMV_WAVES = 4;
constexpr int GEMV_MAXB = 8;
constexpr int GEMV_MAXK = 2048;   // K <= 512 * GEMV_KC
constexpr int GEMV_KC = GEMV_MAXK / 512;

template <typename T, int NB>
__global__ __launch_bounds__(256) void gemv_kernel(GemvBatch g, const float *x, int K, int silu_in) {
  const int prob = blockIdx.y;
  const int N = g.N[prob];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * GEMV_WAVES + wave) * GEMV_ROWS;
  if (row0 >= N) return;
  const int nkc = (K + 511) / 512;   // k-chunks of 8 per lane
  float fx[NB][GEMV_KC][8];
#pragma unroll
  for (int c = 0; c < GEMV_KC; ++c) {
    const int k = c * 512 + lane * 8;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = 0.f;
        if (c < nkc && k + e < K) {
          v = x[(int64_t)b * K + k + e];
          v = silu_in ? silu_f(v) : v;
        }
        fx[b][c][e] = v;
      }
  }
  const T *W = (const T *)g.W[prob];
  const T *bias = (const T *)g.bias[prob];
  float acc[GEMV_ROWS][NB];
#pragma unroll
  for (int r = 0; r < GEMV_ROWS; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
#pragma unroll
  for (int c = 0; c < GEMV_KC; ++c) {
    if (c >= nkc) break;
    const int k = c * 512 + lane * 8;
    if (k >= K) break;
    float w[GEMV_ROWS][8];
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r) {
      const int n = row0 + r < N ? row0 + r : N - 1;
      const T *wr = W + (int64_t)n * K + k;
      if constexpr (sizeof(T) == 2) {
        const bf16x8 wv = *(const bf16x8 *)wr;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[r][e] = (float)wv[e];
      } else {
        const float4 a0 = *(const float4 *)wr, a1 = *(const float4 *)(wr + 4);
        w[r][0] = a0.x; w[r][1] = a0.y; w[r][2] = a0.z; w[r][3] = a0.w;
        w[r][4] = a1.x; w[r][5] = a1.y; w[r][6] = a1.z; w[r][7] = a1.w;
      }
    }
#pragma unroll
    for (int r = 0; r < GEMV_ROWS; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][b] = fmaf(w[r][e], fx[b][c][e], acc[r][b]);
  }
#pragma unroll
  for (int r = 0; r < GEMV_ROWS; ++r) {
    const int n = row0 + r;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = wave_sum(acc[r][b]);
      if (lane == 0 && n < N) g.y[prob][(int64_t)b * g.y_stride[prob] + n] = v + (bias ? to_f32(bias[n]) : 0.f);
    }
  }
}

template <typename T, int NB>
hipError_t gemv_run(const GemvBatch &g, const float *x, int K, bool silu_in, hipStream_t st) {
  int maxN = 0;
  for (int i = 0; i < g.nprob; ++i) maxN = g.N[i] > maxN ? g.N[i] : maxN;
  const int rows_per_block = GEMV_WAVES * GEMV_ROWS;
  dim3 grid((maxN + rows_per_block - 1) / rows_per_block, g.nprob);
  hipLaunchKernelGGL((gemv_kernel<T, NB>), grid, dim3(256), 0, st, g, x, K, silu_in ? 1 : 0);
  return hipGetLastError();
}

// bf16 weights: a persistent grid (GEMV_BLOCKS_PER_CU blocks per CU) walks
// the rows of all problems of the batch as one index space in groups of
// GEMV_RG rows, group g going to wave g mod (waves of the grid), so at any
// time the grid streams one contiguous stretch of the weights.  The block
// stages f(x) for all its samples in LDS once (f is SiLU when silu_in).  A
// wave takes one group at a time with its 16-byte weight loads for all KC
// k-chunks (lane l owns k = 512 c + 8 l .. + 7) in flight together, loaded
// non-temporally (each weight is read once per call); f(x) comes from LDS
// as it is used, so few VGPRs are live and several waves fit per SIMD.
// Measured on MI355X for the 24 AdaLN matrices of 12 blocks (680 MB of
// weights, B = 2): 108 us per launch (6.3 TB/s) against 138 us with
// ordinary loads and a contiguous run of rows per wave.  The RG x NB lane
// partials are reduced by a transposing butterfly: every exchange step
// halves the values a lane holds, so the sums cost about RG x NB shuffles
// instead of 6 each.
constexpr int GEMV_RG = 4;               // rows per group (loads in flight together)
constexpr int GEMV_BLOCKS_PER_CU = 4;

template <int N>
struct pow2_ceil { static constexpr int v = N <= 1 ? 1 : 2 * pow2_ceil<(N + 1) / 2>::v; };
template <>
struct pow2_ceil<1> { static constexpr int v = 1; };

__device__ __forceinline__ bf16x8 load_weights_nt(const bf16 *p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4 *)p));
}

template <int NB, int KC>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(GemvBatch g, const float *x, int K, int silu_in,
                                                        int total_rows) {
  __shared__ __attribute__((aligned(16))) float sx[NB * GEMV_MAXK];
  for (int i = threadIdx.x; i < NB * K; i += 256) {
    const float v = x[i];
    sx[i] = silu_in ? silu_f(v) : v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r_begin = (blockIdx.x * GEMV_WAVES + wave) * GEMV_RG;
  const int r_step = gridDim.x * GEMV_WAVES * GEMV_RG;
  const int r_end = total_rows;
  if (r_begin >= r_end) return;
  // problem of the wave's current row (rows only increase along the walk)
  int prob = 0, pbase = 0;
  constexpr int NV = GEMV_RG * NB, VP = pow2_ceil<NV>::v;
  static_assert(VP <= 64, "values per lane");
#pragma unroll 1
  for (int r0 = r_begin; r0 < r_end; r0 += r_step) {
    // each row's problem and row inside it (rows past the end repeat the last)
    int rp[GEMV_RG], rn[GEMV_RG];
#pragma unroll
    for (int r = 0; r < GEMV_RG; ++r) {
      const int row = min(r0 + r, r_end - 1);
      while (prob + 1 < g.nprob && row >= pbase + g.N[prob]) pbase += g.N[prob++];
      rp[r] = prob;
      rn[r] = row - pbase;
    }
    bf16x8 wv[KC][GEMV_RG];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = c * 512 + lane * 8;
#pragma unroll
      for (int r = 0; r < GEMV_RG; ++r)
        wv[c][r] = k < K ? load_weights_nt((const bf16 *)g.W[rp[r]] + (int64_t)rn[r] * K + k) : bf16x8{};
    }
    float v[VP];
#pragma unroll
    for (int i = 0; i < VP; ++i) v[i] = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int k = c * 512 + lane * 8;
      if (k >= K) break;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 x0 = *(const float4 *)(sx + b * K + k), x1 = *(const float4 *)(sx + b * K + k + 4);
        const float xf[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int r = 0; r < GEMV_RG; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[r * NB + b] = fmaf((float)wv[c][r][e], xf[e], v[r * NB + b]);
      }
    }
    // transposing butterfly: at the step with offset o a lane keeps the
    // upper or lower half of its values (by lane bit o), each summed with
    // its partner's copy
    int o = 32;
#pragma unroll
    for (int cnt = VP; cnt > 1; cnt >>= 1) {
      const bool hi = lane & o;
#pragma unroll
      for (int i = 0; i < cnt / 2; ++i) {
        const float send = hi ? v[i] : v[i + cnt / 2];
        const float keep = hi ? v[i + cnt / 2] : v[i];
        v[i] = keep + __shfl_xor(send, o);
      }
      o >>= 1;
    }
    for (int oo = o; oo >= 1; oo >>= 1) v[0] += __shfl_xor(v[0], oo);
    // now every aligned group of 2 o lanes holds one full sum; its index is
    // the sum of the halves kept (VP / 2 for lane bit 32, VP / 4 for 16, ...)
    if ((lane & (2 * o - 1)) == 0) {
      int idx = 0, w = VP / 2;
#pragma unroll
      for (int oo = 32; oo > o; oo >>= 1, w >>= 1) idx += (lane & oo) ? w : 0;
      if (idx < NV) {
        const int r = idx / NB, b = idx - r * NB;
        if (r0 + r < r_end) {
          const bf16 *bias = (const bf16 *)g.bias[rp[r]];
          g.y[rp[r]][(int64_t)b * g.y_stride[rp[r]] + rn[r]] = v[0] + (bias ? (float)bias[rn[r]] : 0.f);
        }
      }
    }
  }
}

template <int NB, int KC>
hipError_t gemv_bf16_run(const GemvBatch &g, const float *x, int K, bool silu_in, hipStream_t st) {
  int total = 0;
  for (int i = 0; i < g.nprob; ++i) total += g.N[i];
  if (total <= 0) return hipSuccess;
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cus = c;
  }
  // no more blocks than there are row groups
  const int groups = (total + GEMV_RG - 1) / GEMV_RG;
  const int need = (groups + GEMV_WAVES - 1) / GEMV_WAVES;
  const int blocks = need < cus * GEMV_BLOCKS_PER_CU ? need : cus * GEMV_BLOCKS_PER_CU;
  hipLaunchKernelGGL((gemv_bf16_kernel<NB, KC>), dim3(blocks), dim3(256), 0, st, g, x, K, silu_in ? 1 : 0, total);
  return hipGetLastError();
}

template <int NB>
hipError_t gemv_bf16_kc(const GemvBatch &g, const float *x, int K, bool silu_in, hipStream_t st) {
  switch ((K + 511) / 512) {
    case 1: return gemv_bf16_run<NB, 1>(g, x, K, silu_in, st);
    case 2: return gemv_bf16_run<NB, 2>(g, x, K, silu_in, st);
    case 3: return gemv_bf16_run<NB, 3>(g, x, K, silu_in, st);
    default: return gemv_bf16_run<NB, 4>(g, x, K, silu_in, st);
  }
}

template <typename T, int NB>
hipError_t gemv_pick(const GemvBatch &g, const float *x, int K, bool silu_in, hipStream_t st) {
  if constexpr (sizeof(T) == 2) return gemv_bf16_kc<NB>(g, x, K, silu_in, st);
  else return gemv_run<T, NB>(g, x, K, silu_in, st);
}

template <typename T>
hipError_t gemv_dispatch(const GemvBatch &g, const float *x, int B, int K, bool silu_in, hipStream_t st) {
  // batches larger than 8 run as several launches on row offsets of x / y
  for (int b0 = 0; b0 < B; b0 += GEMV_MAXB) {
    const int nb = B - b0 < GEMV_MAXB ? B - b0 : GEMV_MAXB;
    GemvBatch gg = g;
    for (int i = 0; i < g.nprob; ++i) gg.y[i] = g.y[i] + (int64_t)b0 * g.y_stride[i];
    const float *xx = x + (int64_t)b0 * K;
    hipError_t e;
    switch (nb) {
      case 1: e = gemv_pick<T, 1>(gg, xx, K, silu_in, st); break;
      case 2: e = gemv_pick<T, 2>(gg, xx, K, silu_in, st); break;
      case 3: e = gemv_pick<T, 3>(gg, xx, K, silu_in, st); break;
      case 4: e = gemv_pick<T, 4>(gg, xx, K, silu_in, st); break;
      case 5: e = gemv_pick<T, 5>(gg, xx, K, silu_in, st); break;
      case 6: e = gemv_pick<T, 6>(gg, xx, K, silu_in, st); break;
      case 7: e = gemv_pick<T, 7>(gg, xx, K, silu_in, st); break;
      default: e = gemv_pick<T, 8>(gg, xx, K, silu_in, st); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------ timestep features
__global__ void timestep_kernel(const float *t, float *phi, int B, int dim, float t_scale) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int half = dim / 2;
  if (i >= B * half) return;
  const int b = i / half, k = i % half;
  // w_k = 10000^(-k/half), computed in double so the phase of t_scale * t
  // (up to 1000 rad) keeps full float accuracy
  const double w = exp(-(double)k / (double)half * log(10000.0));
  const double arg = (double)t_scale * (double)t[b] * w;
  phi[(int64_t)b * dim + k] = (float)cos(arg);
  phi[(int64_t)b * dim + half + k] = (float)sin(arg);
}

// ------------------------------------------------ text feature RMSNorm
// One block per token row; wave w normalises layers w, w+4, ...  When the
// layer width F splits into 16-byte chunks and a lane's share of them fits
// TXT_CHUNKS, the lane loads its chunks once (16 bytes each) and keeps them
// in registers for the second pass; otherwise element by element.
constexpr int TXT_CHUNKS = 8;

template <typename T>
__global__ __launch_bounds__(256) void txt_norm_kernel(const T *feats, const T *gain, T *out, int layers, int F,
                                                       float eps) {
  constexpr int VEC = 16 / sizeof(T);
  typedef T vecT __attribute__((ext_vector_type(VEC)));
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = F % VEC == 0 ? F / VEC : 0;
  const bool vec = nch > 0 && nch <= 64 * TXT_CHUNKS;
  for (int l = wave; l < layers; l += 4) {
    const T *x = feats + ((int64_t)row * layers + l) * F;
    T *y = out + ((int64_t)row * layers + l) * F;
    const T *g = gain + (int64_t)l * F;
    if (vec) {
      vecT v[TXT_CHUNKS];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < TXT_CHUNKS; ++c) {
        const int ch = c * 64 + lane;
        if (ch < nch) {
          v[c] = *(const vecT *)(x + ch * VEC);
#pragma unroll
          for (int e = 0; e < VEC; ++e) ss += to_f32(v[c][e]) * to_f32(v[c][e]);
        }
      }
      ss = wave_sum(ss);
      const float r = rsqrtf(ss / (float)F + eps);
#pragma unroll
      for (int c = 0; c < TXT_CHUNKS; ++c) {
        const int ch = c * 64 + lane;
        if (ch < nch) {
          const vecT gv = *(const vecT *)(g + ch * VEC);
          vecT o;
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = from_f32<T>(to_f32(v[c][e]) * r * to_f32(gv[e]));
          *(vecT *)(y + ch * VEC) = o;
        }
      }
      continue;
    }
    float ss = 0.f;
    for (int i = lane; i < F; i += 64) {
      const float v = to_f32(x[i]);
      ss += v * v;
    }
    ss = wave_sum(ss);
    const float r = rsqrtf(ss / (float)F + eps);
    for (int i = lane; i < F; i += 64) y[i] = from_f32<T>(to_f32(x[i]) * r * to_f32(g[i]));
  }
}

// ------------------------------------------------ CFG + Euler
template <typename TL>
__global__ void flow_step_kernel(float *x, const float *vc, const float *vu, int64_t n, float dt, float s,
                                 TL *lowp) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float c = vc[i];
    const float v = vu ? vu[i] + s * (c - vu[i]) : c;
    const float xn = x[i] + dt * v;
    x[i] = xn;
    if (lowp) lowp[i] = from_f32<TL>(xn);
  }
}

// Norm-rescaled CFG + Euler (Lens blog, "Exploring Image Editing"): one wave
// per token of C channels; comb = u + s (c - u), rescaled by |c| / |comb|
// (left as is where |comb| = 0), then x += dt * comb.
template <typename TL>
__global__ __launch_bounds__(256) void flow_step_rescaled_kernel(float *x, const float *vc, const float *vu,
                                                                 int64_t ntok, int C, float dt, float s, TL *lowp) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= ntok) return;
  const int64_t base = tok * C;
  float nc = 0.f, nb = 0.f;
  for (int ch = lane; ch < C; ch += 64) {
    const float c = vc[base + ch];
    const float v = vu ? vu[base + ch] + s * (c - vu[base + ch]) : c;
    nc = fmaf(c, c, nc);
    nb = fmaf(v, v, nb);
  }
  nc = wave_sum(nc);
  nb = wave_sum(nb);
  const float f = nb > 0.f ? sqrtf(nc) / sqrtf(nb) : 1.f;
  for (int ch = lane; ch < C; ch += 64) {
    const float c = vc[base + ch];
    const float v = vu ? vu[base + ch] + s * (c - vu[base + ch]) : c;
    const float xn = x[base + ch] + dt * (v * f);
    x[base + ch] = xn;
    if (lowp) lowp[base + ch] = from_f32<TL>(xn);
  }
}

// ------------------------------------------------ MX fp8 quantization
// One thread per 8 consecutive elements; the 4 threads of a 32-block are
// consecutive lanes (scale exponent and element codes: mx_exponent,
// mx_pack4).  Scales row-major ([rows][cols / 32]) or, with slabs,
// slab-major (mx_scale_index).
template <typename T>
__global__ __launch_bounds__(256) void mx_quant_kernel(MxQuantProblem p0, MxQuantProblem p1, int cols, bool slabs) {
  const int64_t groups_per_row = cols / 8;
  const int64_t g0 = p0.rows * groups_per_row;
  int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool second = g >= g0;
  const MxQuantProblem &p = second ? p1 : p0;
  if (second) g -= g0;
  const bool live = g < p.rows * groups_per_row;
  const int64_t gi = live ? g : 0;
  float v[8];
  if constexpr (sizeof(T) == 2) {
    const bf16x8 w = live ? *((const bf16x8 *)p.src + gi) : bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)w[e];
  } else {
    float4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (live) {
      a = *((const float4 *)p.src + 2 * gi);
      b = *((const float4 *)p.src + 2 * gi + 1);
    }
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int ex = mx_exponent(amax);
  if (!live) return;
  const unsigned lo = mx_pack4(v[0], v[1], v[2], v[3], ex), hi = mx_pack4(v[4], v[5], v[6], v[7], ex);
  *((uint2 *)p.q + gi) = make_uint2(lo, hi);
  if ((gi & 3) == 0) {
    const int64_t r = gi / groups_per_row, kb = (gi - r * groups_per_row) >> 2;
    ((unsigned char *)p.scale)[slabs ? mx_scale_index(r, kb, p.rows) : gi >> 2] = (unsigned char)(ex + 127);
  }
}

}  // namespace

hipError_t launch_mx_quant(const MxQuantProblem *p, int nprob, int cols, bool src_bf16, bool slabs,
                           hipStream_t stream) {
  if (cols <= 0 || cols % (slabs ? 128 : 32)) return hipErrorInvalidValue;
  MxQuantProblem p1 = nprob > 1 ? p[1] : MxQuantProblem{};
  if (nprob < 2) p1.rows = 0;
  const int64_t groups = (p[0].rows + p1.rows) * (cols / 8);
  if (groups == 0) return hipSuccess;
  const int64_t blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (src_bf16)
    hipLaunchKernelGGL(mx_quant_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, p[0], p1, cols, slabs);
  else
    hipLaunchKernelGGL(mx_quant_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, p[0], p1, cols, slabs);
  return hipGetLastError();
}

hipError_t launch_norm_modulate(const NormModProblem *p, int nprob, int D, float eps, bool bf16_path,
                                hipStream_t stream, bool mx_out) {
  NormModProblem p1 = nprob > 1 ? p[1] : NormModProblem{};
  if (nprob < 2) p1.rows = 0;
  const int rows = p[0].rows + p1.rows;
  if (rows == 0) return hipSuccess;
  const int rw = norm_rw(mx_out);
  const int split0 = (p[0].rows + rw - 1) / rw * rw;
  const int waves = split0 / rw + (p1.rows + rw - 1) / rw;
  dim3 grid((waves + 3) / 4);
  if (mx_out && (!p[0].out_scale || (nprob > 1 && p1.rows > 0 && !p1.out_scale))) return hipErrorInvalidValue;
#define NORM_CASE(g)                                                                                     \
  case g:                                                                                                \
    if (mx_out)                                                                                          \
      hipLaunchKernelGGL((norm_modulate_kernel<float, g, true>), grid, dim3(256), 0, stream, p[0], p1, split0, eps); \
    else if (bf16_path)                                                                                  \
      hipLaunchKernelGGL((norm_modulate_kernel<bf16, g>), grid, dim3(256), 0, stream, p[0], p1, split0, eps);   \
    else                                                                                                 \
      hipLaunchKernelGGL((norm_modulate_kernel<float, g>), grid, dim3(256), 0, stream, p[0], p1, split0, eps);  \
    break;
  switch (D / 256) {
    NORM_CASE(1) NORM_CASE(2) NORM_CASE(3) NORM_CASE(4) NORM_CASE(5) NORM_CASE(6) NORM_CASE(7) NORM_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef NORM_CASE
  return hipGetLastError();
}

namespace {

// (cos, sin) of every joint position and rotation pair, with the same
// angle arithmetic as qknorm_rope_kernel.
__global__ void rope_table_kernel(const int32_t *pos_img, const int32_t *pos_txt, int S_img, int S_txt, int axes0,
                                  int axes1, int axes2, float theta, float2 *rope) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (S_img + S_txt) * 32) return;
  const int jp = idx >> 5, i = idx & 31, d = 2 * i;
  const int32_t *pos = jp < S_img ? pos_img + 3 * jp : pos_txt + 3 * (jp - S_img);
  float pa, j, w;
  if (d < axes0) {
    pa = (float)pos[0]; j = (float)(d / 2); w = (float)axes0;
  } else if (d < axes0 + axes1) {
    pa = (float)pos[1]; j = (float)((d - axes0) / 2); w = (float)axes1;
  } else {
    pa = (float)pos[2]; j = (float)((d - axes0 - axes1) / 2); w = (float)axes2;
  }
  const float l2t = log2f(theta);
  const float ang = pa * exp2f(-2.f * j / w * l2t);
  float sn, cs;
  sincosf(ang, &sn, &cs);
  rope[idx] = make_float2(cs, sn);
}

// one thread per 8 bf16 of a padding row of Q, K and V
__global__ void zero_pad_kernel(bf16 *Q, bf16 *K, bf16 *V, int S, int S_pad, int64_t n8) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const int npad = S_pad - S;
  const int64_t bh = i / ((int64_t)npad * 8), rem = i % ((int64_t)npad * 8);
  const int64_t off = (bh * S_pad + S + rem / 8) * 64 + (rem % 8) * 8;
  const bf16x8 z = {};
  *(bf16x8 *)(Q + off) = z;
  *(bf16x8 *)(K + off) = z;
  *(bf16x8 *)(V + off) = z;
}

}  // namespace

hipError_t launch_rope_table(const int32_t *pos_img, const int32_t *pos_txt, int S_img, int S_txt, int axes0,
                             int axes1, int axes2, float theta, float2 *rope, hipStream_t stream) {
  const int n = (S_img + S_txt) * 32;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, pos_img, pos_txt, S_img, S_txt,
                     axes0, axes1, axes2, theta, rope);
  return hipGetLastError();
}

hipError_t launch_zero_pad_rows(void *Q, void *K, void *V, int B, int H, int S, int S_pad, hipStream_t stream) {
  const int64_t n8 = (int64_t)B * H * (S_pad - S) * 8;
  if (n8 <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_pad_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, (bf16 *)Q, (bf16 *)K,
                     (bf16 *)V, S, S_pad, n8);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(const QkRopeArgs &a, bool bf16_path, hipStream_t stream) {
  dim3 grid(a.S_pad / 64, a.H, a.B);
  if (bf16_path)
    hipLaunchKernelGGL(qknorm_rope_kernel<bf16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(qknorm_rope_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvBatch &g, const float *x, int B, int K, bool silu_in, bool bf16_path,
                       hipStream_t stream) {
  if (g.nprob == 0 || B == 0) return hipSuccess;
  return bf16_path ? gemv_dispatch<bf16>(g, x, B, K, silu_in, stream)
                   : gemv_dispatch<float>(g, x, B, K, silu_in, stream);
}

hipError_t launch_timestep_features(const float *t, float *phi, int B, int dim, float t_scale,
                                    hipStream_t stream) {
  const int n = B * (dim / 2);
  hipLaunchKernelGGL(timestep_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, t, phi, B, dim, t_scale);
  return hipGetLastError();
}

hipError_t launch_txt_norm(const void *feats, const void *gain, void *out, int rows, int layers, int F, float eps,
                           bool bf16_path, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (bf16_path)
    hipLaunchKernelGGL(txt_norm_kernel<bf16>, dim3(rows), dim3(256), 0, stream, (const bf16 *)feats,
                       (const bf16 *)gain, (bf16 *)out, layers, F, eps);
  else
    hipLaunchKernelGGL(txt_norm_kernel<float>, dim3(rows), dim3(256), 0, stream, (const float *)feats,
                       (const float *)gain, (float *)out, layers, F, eps);
  return hipGetLastError();
}

hipError_t launch_flow_step(float *x, const float *vc, const float *vu, int64_t n, float dt, float s, void *lowp,
                            int lowp_bf16, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (lowp_bf16)
    hipLaunchKernelGGL(flow_step_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, x, vc, vu, n, dt, s,
                       (bf16 *)lowp);
  else
    hipLaunchKernelGGL(flow_step_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, x, vc, vu, n, dt, s,
                       (float *)lowp);
  return hipGetLastError();
}

hipError_t launch_flow_step_rescaled(float *x, const float *vc, const float *vu, int64_t ntok, int C, float dt,
                                     float s, void *lowp, int lowp_bf16, hipStream_t stream) {
  if (ntok <= 0) return hipSuccess;
  const int64_t blocks = (ntok + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (lowp && lowp_bf16)
    hipLaunchKernelGGL(flow_step_rescaled_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, x, vc, vu, ntok,
                       C, dt, s, (bf16 *)lowp);
  else
    hipLaunchKernelGGL(flow_step_rescaled_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, x, vc, vu,
                       ntok, C, dt, s, (float *)lowp);
  return hipGetLastError();
}

}  // namespace lens

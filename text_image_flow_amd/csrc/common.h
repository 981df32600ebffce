// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lens {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16-byte staging

// float <-> bf16 with round-to-nearest-even (NaN stays NaN).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// SiLU(x) = x / (1 + e^-x), with the hardware reciprocal (1 ulp) in place of
// an IEEE division (a dozen instructions more per element in the GEMM
// epilogues, where the result is rounded to bf16 anyway).  e^-x = inf gives
// x * 0 = -0, as the division does; NaN stays NaN.
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// ---------------------------------------------------------------- MX fp8
// MX-style fp8 with a non-saturating scale (the block-scaled low-precision
// weights of the Lens-3.8B-4bit article, section 4): e4m3 elements, one E8M0
// power-of-two scale per 32 consecutive elements.  Unlike the OCP MX v1.0
// rule (scale exponent floor(log2 amax) - 8, saturating the few elements
// that then exceed 448), the scale here is the tightest one under which no
// element saturates.  Scale exponent of a block with largest magnitude amax: the
// smallest e with amax <= 448 * 2^e, read off amax's fp32 bits (amax =
// 1.f * 2^E: e = E - 8, plus one when f > 0.75), clamped to [-127, 127]; an
// all-zero block takes -127.  The byte is e + 127.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (amax == 0.f) return -127;
  const unsigned b = __float_as_uint(amax);
  const int ex = (int)(b >> 23) - 127 - 8 + ((b & 0x7fffff) > 0x600000 ? 1 : 0);
  return ex < -127 ? -127 : (ex > 127 ? 127 : ex);
}

// Byte position of the scale of (row, 32-block kb) in the slab-major scale
// layout the fp8 GEMM reads: [K / 128][rows][4], i.e. for every 128-wide
// slab of the reduction axis each row's 4 block scales form one 4-byte word.
__device__ __host__ __forceinline__ int64_t mx_scale_index(int64_t row, int64_t kb, int64_t rows) {
  return ((kb >> 2) * rows + row) * 4 + (kb & 3);
}

// Four elements of one block (scale exponent ex) as four e4m3 bytes, first
// element in the low byte: x / 2^ex rounded to the nearest e4m3 value, ties
// to even, subnormals in steps of 2^-9 (|x / 2^ex| <= 448 by the choice of
// ex).  The gfx950 conversion v_cvt_pk_fp8_f32 does exactly this rounding:
// checked on MI355X against an integer encoder of the rule on every fp32
// bit pattern with magnitude in [2^-20, 448], both signs (smaller
// magnitudes round to zero in both).
__device__ __forceinline__ unsigned mx_pack4(float a, float b, float c, float d, int ex) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(a, -ex), ldexpf(b, -ex), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(c, -ex), ldexpf(d, -ex), w, true);
  return (unsigned)w;
}

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `stream` and return hipSuccess or the launch error.

enum Epilogue {
  EPI_STORE = 0,     // C = acc + bias                    (C in act type)
  EPI_STORE_F32 = 1, // C = acc + bias                    (C float)
  EPI_GATED = 2,     // H += gate[m / rows_per_gate] * (acc + bias)   (H float)
  EPI_SWIGLU = 3,    // C = silu(acc1 + b1) * (acc3 + b3), B rows from w1 and w3
  EPI_QKV = 4,       // y = acc + bias split into per-head q | k | v (QkvOut; bf16 only):
                     // q, k RMS-normed with gain and rotated (RoPE), q scaled,
                     // all three written to the joint [B, H, S_pad, 64] layout
  EPI_SWIGLU_MX = 5  // EPI_SWIGLU written as MX fp8: C e4m3 [M, N], C_scale E8M0 slab-major
                     // (mx_scale_index; launch_gemm_fp8 only)
};

// One GEMM problem: C[M, N] = A[M, K] . W[N, K]^T (+ epilogue).
struct GemmProblem {
  const void *A;       // [M, K] act type
  const void *W;       // [N, K] act type (for SWIGLU: w1)
  const void *W3;      // SWIGLU only: w3 [N, K]
  const void *bias;    // [N] or NULL (SWIGLU: b1)
  const void *bias3;   // SWIGLU only: b3 or NULL
  void *C;             // output (see Epilogue)
  const float *gate;   // EPI_GATED: gate rows, gate[(m / rows_per_gate) * gate_stride + n]
  int64_t gate_stride;
  int32_t rows_per_gate;
  int32_t M, N, K;
  // MX fp8 operands (launch_gemm_fp8 only): A, W, W3 hold e4m3 bytes and
  // these their E8M0 scales, one byte per 32 elements along K, slab-major
  // ([K / 128][rows][4], see mx_scale_index)
  const void *A_scale, *W_scale, *W3_scale;
  void *C_scale;       // EPI_SWIGLU_MX: output scales
};

// Outputs of the QKV epilogue.  Problem 0 holds the image rows of the batch
// (b * S_img + p -> joint position p), problem 1 the text rows (b * S_txt + p
// -> joint position S_img + p).  rope: [S_img + S_txt][32] (cos, sin) of
// every joint position and rotation pair.
struct QkvOut {
  void *Q, *K, *V;                      // [B, H, S_pad, 64] bf16
  const void *q_gain[2], *k_gain[2];    // per problem, [64] bf16
  const float2 *rope;
  int32_t S_img, S_txt, S_pad, H;
  float eps, q_scale;
};

// Grouped launch of up to 2 problems that share N, K and the epilogue
// (qo: EPI_QKV only).
hipError_t launch_gemm(int epi, bool bf16_path, const GemmProblem *probs, int nprob, hipStream_t stream,
                       const QkvOut *qo = nullptr);
// Kernels the calling thread's last launch_gemm / launch_gemm_fp8 issued.
int gemm_kernels_launched();

// The same grouped GEMM on MX fp8 operands (e4m3 elements, E8M0 scales per
// 32 along K; K % 128 == 0); the epilogues are those of the bf16 path.
hipError_t launch_gemm_fp8(int epi, const GemmProblem *probs, int nprob, hipStream_t stream,
                           const QkvOut *qo = nullptr);

// MX fp8 quantization along rows: src [rows, cols] (bf16 or f32, cols % 32
// == 0) -> q [rows, cols] e4m3 bytes and E8M0 scales, one per 32 elements,
// row-major [rows][cols / 32] or, with slabs (cols % 128 == 0), slab-major
// (mx_scale_index); per block of 32 the tightest power-of-two scale that
// keeps every element within +-448, elements rounded to nearest (ties to
// even).  Up to 2 problems in one launch (rows1 = 0 for one).
struct MxQuantProblem {
  const void *src;
  void *q, *scale;
  int64_t rows;
};
hipError_t launch_mx_quant(const MxQuantProblem *p, int nprob, int cols, bool src_bf16, bool slabs,
                           hipStream_t stream);

// RoPE table of the joint sequence: rope[j][i] = (cos, sin) of pos(j)[axis] *
// theta^(-2 i' / axis_dim) for rotation pair i (pairs 0 .. axes0/2 - 1 on axis
// 0, then axis 1, then axis 2; i' = index inside the axis), the angles
// computed exactly as the QK-norm/RoPE kernel does.
hipError_t launch_rope_table(const int32_t *pos_img, const int32_t *pos_txt, int S_img, int S_txt, int axes0,
                             int axes1, int axes2, float theta, float2 *rope, hipStream_t stream);
// Zero rows S .. S_pad - 1 of every (b, h) of the joint Q, K, V (bf16).
hipError_t launch_zero_pad_rows(void *Q, void *K, void *V, int B, int H, int S, int S_pad, hipStream_t stream);

// Joint attention.  Q, K, V: [B, H, S_pad, 64] (act type), rows >= S zero.
// bf16 path: Q pre-scaled by scale * log2(e) (QkRopeArgs);
// fp32 path: plain Q, scale applied inside.
// Output rows p < S_img go to O_img[(b*S_img + p), h*64 + d], rows
// S_img <= p < S_img + S_txt to O_txt[(b*S_txt + p - S_img), ...].
// Valid keys of sample b: [0, S_img + clamp(txt_len[b], 0, S_txt)).
struct AttnArgs {
  const void *Q, *K, *V;
  void *O_img, *O_txt;
  const int32_t *txt_len;  // device, [B] or NULL
  int32_t B, H, S_img, S_txt, S_pad;
  float scale;             // 1/sqrt(head_dim)
  // bf16 path: the [64] q/k RMSNorm gains of both streams (q_img, k_img,
  // q_txt, k_txt), from which the kernel bounds every score; NULL: no bound
  const void *gain[4];
  // bf16 path, optional: O as MX fp8 rows instead (e4m3 [B*S, H*64], E8M0
  // scales slab-major over the B*S rows of each stream); with O8_img set,
  // O_img / O_txt are not written
  void *O8_img, *O8_txt, *OS_img, *OS_txt;
};
hipError_t launch_attention(const AttnArgs &a, bool bf16_path, hipStream_t stream);

// Per-row RMSNorm (no gain) + modulation, both streams in one launch.
// out[r] = h[r] / rms(h[r]) * (1 + scale[b]) + shift[b], b = r / rows_per_sample.
struct NormModProblem {
  const float *h;
  void *out;
  const float *shift, *scale;  // [B, D] rows, stride mod_stride
  int64_t mod_stride;
  int32_t rows, rows_per_sample;
  void *out_scale;             // mx_out: E8M0 scales, slab-major over rows (out: e4m3 [rows, D])
};
hipError_t launch_norm_modulate(const NormModProblem *p, int nprob, int D, float eps, bool bf16_path,
                                hipStream_t stream, bool mx_out = false);

// QK RMSNorm + RoPE + joint layout.  qkv_img [B*S_img, 3D], qkv_txt [B*S_txt, 3D].
// q_scale multiplies q after RoPE (the bf16 attention kernel takes Q in
// log2 units: scale * log2(e)).  Q, K, V out: [B, H, S_pad, 64], rows >= S
// zero.
struct QkRopeArgs {
  const void *qkv_img, *qkv_txt;
  const void *qg_img, *kg_img, *qg_txt, *kg_txt;  // [64] act type
  const int32_t *pos_img, *pos_txt;               // [S, 3]
  void *Q, *K, *V;
  int32_t B, H, S_img, S_txt, S_pad;
  int32_t axes0, axes1, axes2;
  float theta, eps;
  float q_scale;
};
hipError_t launch_qknorm_rope(const QkRopeArgs &a, bool bf16_path, hipStream_t stream);

// Skinny GEMM (GEMV over a small batch): y[b, n] = sum_k f(x[b, k]) W[n, k] + bias[n],
// f = SiLU when silu_in, else identity.  x float [B, K], y float [B, N] rows at
// y + b * y_stride.  Up to GEMV_MAX_PROBS problems share x, B and K (25: the
// 96 AdaLN matrices of 48 blocks and the final layer's modulation go out in
// four launches; the batch, passed by value, stays under 1 KB of kernel
// arguments).
constexpr int GEMV_MAX_PROBS = 25;
struct GemvBatch {
  const void *W[GEMV_MAX_PROBS];
  const void *bias[GEMV_MAX_PROBS];
  float *y[GEMV_MAX_PROBS];
  int32_t N[GEMV_MAX_PROBS];
  int64_t y_stride[GEMV_MAX_PROBS];
  int32_t nprob;
};
hipError_t launch_gemv(const GemvBatch &g, const float *x, int B, int K, bool silu_in, bool bf16_path,
                       hipStream_t stream);

// Sinusoidal timestep features: phi[b] = [cos(scale t w_k) | sin(scale t w_k)].
hipError_t launch_timestep_features(const float *t, float *phi, int B, int dim, float t_scale,
                                    hipStream_t stream);

// Text input: per encoder layer RMSNorm with gain; rows of layers * F.
hipError_t launch_txt_norm(const void *feats, const void *gain, void *out, int rows, int layers, int F,
                           float eps, bool bf16_path, hipStream_t stream);

// Euler + CFG step on n elements.
hipError_t launch_flow_step(float *x, const float *vc, const float *vu, int64_t n, float dt, float s,
                            void *lowp, int lowp_bf16, hipStream_t stream);
// Euler + norm-rescaled CFG on ntok tokens of C channels.
hipError_t launch_flow_step_rescaled(float *x, const float *vc, const float *vu, int64_t ntok, int C, float dt,
                                     float s, void *lowp, int lowp_bf16, hipStream_t stream);

}  // namespace lens

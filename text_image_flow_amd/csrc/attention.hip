// Joint text+image attention of the MM-DiT block: for every sample and head,
// O = softmax(Q K^T / sqrt(64) + M) V over the sample's image tokens and its
// valid text tokens, no causal mask.  (Lens-Turbo-3.8B-bf16 article, dual
// stream attention: the two streams attend to each other; Lens blog,
// "Exploring Text Encoder": zero-padded text is invisible to the DiT.)
//
// Joint layout per sample: image tokens [0, S_img), text tokens
// [S_img, S_img + S_txt), zero padding up to S_pad (a multiple of 64).  With
// text after image, the key mask is a per-sample key count
// kv_len = S_img + txt_len[b]; the softmax over a permuted key set is the
// same, so this order gives the same result as text-then-image.
//
// bf16 path (flash-style, one pass over K/V):
//   * a wave owns 32 queries; four waves share 64-key K and V^T tiles that
//     are double-buffered in LDS;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: each lane then holds one
//     query (lane & 31) and 32 of the tile's 64 keys, so the row max needs
//     one exchange with the partner lane (lane ^ 32) and the row sum none
//     until the end;
//   * P^T is rounded to bf16 in registers and used directly as the B operand
//     of O^T += V^T P^T (V is stored transposed, [64, S_pad], so V^T
//     fragments are plain LDS reads); O^T keeps one query per lane, so the
//     online-softmax rescale is a per-lane scalar;
//   * exponentials are exp2 of (s * scale * log2 e - m), one FMA per score.
// fp32 path: one thread per query, plain loops (correctness only).
#include "common.h"

namespace lens {

namespace {

constexpr int KV_T = 64;        // keys per tile
constexpr int LROW = 64 + 8;    // LDS row stride (bf16 elements)
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ int kv_count(const AttnArgs &a, int b) {
  int tl = a.S_txt;
  if (a.txt_len) {
    tl = a.txt_len[b];
    tl = tl < 0 ? 0 : (tl > a.S_txt ? a.S_txt : tl);
  }
  return a.S_img + tl;
}

template <typename T>
__device__ __forceinline__ T *out_row(const AttnArgs &a, int b, int p) {
  const int D = a.H * 64;
  if (p < a.S_img) return (T *)a.O_img + ((int64_t)b * a.S_img + p) * D;
  return (T *)a.O_txt + ((int64_t)b * a.S_txt + (p - a.S_img)) * D;
}

__global__ __launch_bounds__(256) void attn_bf16_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sK[2][KV_T * LROW];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][64 * LROW];

  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = a.S_img + a.S_txt;
  const int q0 = blockIdx.x * 128 + wave * 32;
  const int64_t bh = (int64_t)b * a.H + h;
  const bf16 *Qg = (const bf16 *)a.Q + bh * a.S_pad * 64;
  const bf16 *Kg = (const bf16 *)a.K + bh * a.S_pad * 64;
  const bf16 *Vg = (const bf16 *)a.Vt + bh * 64 * a.S_pad;
  const int n_kv = kv_count(a, b);
  const int n_tiles = (n_kv + KV_T - 1) / KV_T;
  const float c = a.scale * LOG2E;

  const int hl = lane >> 5;      // which half of the wave
  const int ql = lane & 31;      // this lane's query within the wave
  // Q^T fragments (B operand): query row, 8 head dims per k-step of 16
  bf16x8 qf[4];
  {
    int qr = q0 + ql;
    qr = qr < S ? qr : S - 1;
    const bf16 *src = Qg + (int64_t)qr * 64 + hl * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *(const bf16x8 *)(src + ks * 16);
  }

  // tile staging: 2 K chunks + 2 V^T chunks of 16 bytes per thread
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const bf16 *k_src0 = Kg + (int64_t)lr * 64 + lc;
  const bf16 *k_src1 = Kg + (int64_t)(lr + 32) * 64 + lc;
  const bf16 *v_src0 = Vg + (int64_t)lr * a.S_pad + lc;
  const bf16 *v_src1 = Vg + (int64_t)(lr + 32) * a.S_pad + lc;
  const int l_off0 = lr * LROW + lc, l_off1 = (lr + 32) * LROW + lc;
  u32x4 rk0 = *(const u32x4 *)k_src0, rk1 = *(const u32x4 *)k_src1;
  u32x4 rv0 = *(const u32x4 *)v_src0, rv1 = *(const u32x4 *)v_src1;
  *(u32x4 *)&sK[0][l_off0] = rk0;
  *(u32x4 *)&sK[0][l_off1] = rk1;
  *(u32x4 *)&sV[0][l_off0] = rv0;
  *(u32x4 *)&sV[0][l_off1] = rv1;

  f32x16 o0 = {}, o1 = {};
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int kv0 = t * KV_T;
    const bool more = t + 1 < n_tiles;
    if (more) {
      const int64_t ko = (int64_t)(kv0 + KV_T) * 64, vo = kv0 + KV_T;
      rk0 = *(const u32x4 *)(k_src0 + ko);
      rk1 = *(const u32x4 *)(k_src1 + ko);
      rv0 = *(const u32x4 *)(v_src0 + vo);
      rv1 = *(const u32x4 *)(v_src1 + vo);
    }
    const bf16 *sKb = sK[buf];
    const bf16 *sVb = sV[buf];

    // S^T for keys kv0 + [0, 32) (s0) and kv0 + [32, 64) (s1)
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 k0 = *(const bf16x8 *)&sKb[ql * LROW + ks * 16 + hl * 8];
      const bf16x8 k1 = *(const bf16x8 *)&sKb[(32 + ql) * LROW + ks * 16 + hl * 8];
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[ks], s1, 0, 0, 0);
    }
    // key index of s0[r]: kv0 + (r/4)*8 + hl*4 + r%4; of s1[r]: that + 32
    if (kv0 + KV_T > n_kv) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = kv0 + (r >> 2) * 8 + hl * 4 + (r & 3);
        if (kv >= n_kv) s0[r] = -INFINITY;
        if (kv + 32 >= n_kv) s1[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    // P^T as bf16 B operands: pb[ks] holds keys ks*16 + (e/4)*8 + hl*4 + e%4
    bf16x8 pb0, pb1, pb2, pb3;
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[e], c, -m_new));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s0[8 + e], c, -m_new));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(s1[e], c, -m_new));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(s1[8 + e], c, -m_new));
      ls += (p0 + p1) + (p2 + p3);
      pb0[e] = (bf16)p0;
      pb1[e] = (bf16)p1;
      pb2[e] = (bf16)p2;
      pb3[e] = (bf16)p3;
    }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= alpha;
      o1[r] *= alpha;
    }

    // O^T[d, q] += V^T[d, kv] P^T[kv, q]; k-slot (hl, e) is key
    // ks*16 + (e/4)*8 + hl*4 + e%4 in both operands.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 pb = ks == 0 ? pb0 : ks == 1 ? pb1 : ks == 2 ? pb2 : pb3;
      const bf16 *r0 = &sVb[ql * LROW + ks * 16 + hl * 4];
      const bf16 *r1 = &sVb[(32 + ql) * LROW + ks * 16 + hl * 4];
      const bf16x4 a0 = *(const bf16x4 *)r0, b0 = *(const bf16x4 *)(r0 + 8);
      const bf16x4 a1 = *(const bf16x4 *)r1, b1 = *(const bf16x4 *)(r1 + 8);
      const bf16x8 v0 = {a0[0], a0[1], a0[2], a0[3], b0[0], b0[1], b0[2], b0[3]};
      const bf16x8 v1 = {a1[0], a1[1], a1[2], a1[3], b1[0], b1[1], b1[2], b1[3]};
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pb, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pb, o1, 0, 0, 0);
    }
    if (more) {
      *(u32x4 *)&sK[buf ^ 1][l_off0] = rk0;
      *(u32x4 *)&sK[buf ^ 1][l_off1] = rk1;
      *(u32x4 *)&sV[buf ^ 1][l_off0] = rv0;
      *(u32x4 *)&sV[buf ^ 1][l_off1] = rv1;
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  const int p = q0 + ql;
  if (p >= S) return;
  bf16 *dst = out_row<bf16>(a, b, p) + h * 64;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    bf16x4 v0, v1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v0[e] = (bf16)(o0[g * 4 + e] * inv);
      v1[e] = (bf16)(o1[g * 4 + e] * inv);
    }
    *(bf16x4 *)(dst + g * 8 + hl * 4) = v0;
    *(bf16x4 *)(dst + 32 + g * 8 + hl * 4) = v1;
  }
}

// ------------------------------------------------------------------- fp32
__global__ __launch_bounds__(64) void attn_f32_simple(AttnArgs a) {
  __shared__ float sK[64][65];
  __shared__ float sV[64][65];  // [d][key]
  const int b = blockIdx.z, h = blockIdx.y;
  const int S = a.S_img + a.S_txt;
  const int p = blockIdx.x * 64 + threadIdx.x;
  const int64_t bh = (int64_t)b * a.H + h;
  const float *Qg = (const float *)a.Q + bh * a.S_pad * 64;
  const float *Kg = (const float *)a.K + bh * a.S_pad * 64;
  const float *Vg = (const float *)a.Vt + bh * 64 * a.S_pad;
  const int n_kv = kv_count(a, b);
  float q[64], o[64];
  const int pr = p < S ? p : S - 1;
  for (int d = 0; d < 64; ++d) {
    q[d] = Qg[(int64_t)pr * 64 + d] * a.scale;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int kv0 = 0; kv0 < n_kv; kv0 += 64) {
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 64) {
      const int r = e / 64, d = e % 64;
      sK[r][d] = Kg[(int64_t)(kv0 + r) * 64 + d];
      sV[r][d] = Vg[(int64_t)r * a.S_pad + kv0 + d];
    }
    __syncthreads();
    const int nk = n_kv - kv0 < 64 ? n_kv - kv0 : 64;
    for (int j = 0; j < nk; ++j) {
      float s = 0.f;
      for (int d = 0; d < 64; ++d) s = fmaf(q[d], sK[j][d], s);
      const float mn = fmaxf(m, s);
      const float al = expf(m - mn);
      const float pv = expf(s - mn);
      l = l * al + pv;
      for (int d = 0; d < 64; ++d) o[d] = o[d] * al + pv * sV[d][j];
      m = mn;
    }
  }
  if (p >= S) return;
  float *dst = out_row<float>(a, b, p) + h * 64;
  for (int d = 0; d < 64; ++d) dst[d] = o[d] / l;
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, bool bf16_path, hipStream_t stream) {
  const int S = a.S_img + a.S_txt;
  if (bf16_path) {
    hipLaunchKernelGGL(attn_bf16_mfma, dim3((S + 127) / 128, a.H, a.B), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_f32_simple, dim3((S + 63) / 64, a.H, a.B), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace lens

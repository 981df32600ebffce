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
//     of O^T += V^T P^T (V stored transposed, [64, S_pad]); O^T keeps one
//     query per lane, so the online-softmax rescale is a per-lane scalar;
//   * Q arrives pre-scaled by scale * log2(e), so p = exp2(s - m);
//   * the grid is flat and XCD-aware (one head's q-blocks share an L2).
// fp32 path: one thread per query, plain loops (correctness only).
#include "common.h"

namespace lens {

namespace {

constexpr int KV_T = 64;        // keys per tile
constexpr int LROW = 64 + 8;    // LDS row stride (bf16 elements)

__device__ __forceinline__ int kv_count(const AttnArgs &a, int b) {
  int tl = a.S_txt;
  if (a.txt_len) {
    tl = a.txt_len[b];
    tl = tl < 0 ? 0 : (tl > a.S_txt ? a.S_txt : tl);
  }
  return a.S_img + tl;
}

// Workgroups are dispatched round-robin over the 8 XCDs.  The grid is flat;
// logical block L = (b, h, q-block) with q-block fastest, and XCD x runs the
// contiguous logical range [x * n / 8, (x + 1) * n / 8), so the q-blocks of
// one head share that XCD's L2 copy of the head's K and V.
__device__ __forceinline__ void attn_block_coords(int nqb, int H, int &qb, int &h, int &b) {
  const int n = gridDim.x;
  int bid = blockIdx.x;
  const int per = n / 8;
  if (bid < per * 8) bid = (bid % 8) * per + bid / 8;
  qb = bid % nqb;
  h = (bid / nqb) % H;
  b = bid / (nqb * H);
}

template <typename T>
__device__ __forceinline__ T *out_row(const AttnArgs &a, int b, int p) {
  const int D = a.H * 64;
  if (p < a.S_img) return (T *)a.O_img + ((int64_t)b * a.S_img + p) * D;
  return (T *)a.O_txt + ((int64_t)b * a.S_txt + (p - a.S_img)) * D;
}

// -------------------------------------------------------------- bf16
// Inputs as the bf16 joint layout above, with two differences the QK-norm
// kernel provides: Q is pre-multiplied by scale * log2(e), so S = Q K^T is
// already in log2 units, and within every 16 keys of V^T the key index has
// bits 2 and 3 swapped, so the 8 keys one lane feeds into a PV k-step are
// contiguous (one 16-byte LDS read per V^T fragment).
//
// A wave owns G groups of 32 queries; every K and V^T fragment read from
// LDS feeds G MFMAs.  The running max is lazy: rows rescale only when a
// tile's max exceeds the running max by more than TAU (log2 units), so
// probabilities stay <= 2^TAU, and most tiles skip the O rescale.  Row sums
// add the bf16-rounded probabilities with v_dot2 (the same values the PV
// MFMA consumes).
constexpr float TAU = 8.0f;

// One KV tile of the v2 kernel for G query groups; MASK handles the last,
// partial tile (keys >= n_kv get probability 0).
template <int G, bool MASK>
__device__ __forceinline__ void attn_tile(const bf16 *sKb, const bf16 *sVb, const bf16x8 (&qf)[G][4],
                                          f32x16 (&o)[G][2], float (&m_run)[G], float (&l_run)[G], int kv0,
                                          int n_kv, int ql, int hl) {
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  // S^T (log2 units) for keys kv0 + [0, 32) (s[g][0]) and kv0 + [32, 64) (s[g][1])
  f32x16 s[G][2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    s[g][0] = f32x16{};
    s[g][1] = f32x16{};
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 k0 = *(const bf16x8 *)&sKb[ql * LROW + ks * 16 + hl * 8];
    const bf16x8 k1 = *(const bf16x8 *)&sKb[(32 + ql) * LROW + ks * 16 + hl * 8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s[g][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[g][ks], s[g][0], 0, 0, 0);
      s[g][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[g][ks], s[g][1], 0, 0, 0);
    }
  }
  if (MASK && kv0 + KV_T > n_kv) {
    // key of s[g][0][r]: kv0 + (r/4)*8 + hl*4 + r%4; of s[g][1][r]: that + 32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = kv0 + (r >> 2) * 8 + hl * 4 + (r & 3);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (kv >= n_kv) s[g][0][r] = -INFINITY;
        if (kv + 32 >= n_kv) s[g][1][r] = -INFINITY;
      }
    }
  }
  bf16x8 pb[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = fmaxf(s[g][0][0], s[g][1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s[g][0][r]), s[g][1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > m_run[g] + TAU)) {
      const float m_new = fmaxf(m_run[g], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
      m_run[g] = m_new;
      l_run[g] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[g][0][r] *= alpha;
        o[g][1][r] *= alpha;
      }
    }
    const float m = m_run[g];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      bf16x2 p0 = {(bf16)__builtin_amdgcn_exp2f(s[g][0][e] - m), (bf16)__builtin_amdgcn_exp2f(s[g][0][e + 1] - m)};
      bf16x2 p1 = {(bf16)__builtin_amdgcn_exp2f(s[g][0][8 + e] - m), (bf16)__builtin_amdgcn_exp2f(s[g][0][9 + e] - m)};
      bf16x2 p2 = {(bf16)__builtin_amdgcn_exp2f(s[g][1][e] - m), (bf16)__builtin_amdgcn_exp2f(s[g][1][e + 1] - m)};
      bf16x2 p3 = {(bf16)__builtin_amdgcn_exp2f(s[g][1][8 + e] - m), (bf16)__builtin_amdgcn_exp2f(s[g][1][9 + e] - m)};
      lsum = __builtin_amdgcn_fdot2_f32_bf16(p0, ones, lsum, false);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(p1, ones, lsum, false);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, lsum, false);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(p3, ones, lsum, false);
      pb[g][0][e] = p0[0]; pb[g][0][e + 1] = p0[1];
      pb[g][1][e] = p1[0]; pb[g][1][e + 1] = p1[1];
      pb[g][2][e] = p2[0]; pb[g][2][e + 1] = p2[1];
      pb[g][3][e] = p3[0]; pb[g][3][e + 1] = p3[1];
    }
    l_run[g] += lsum;
  }
  // O^T += V^T P^T: the permuted V^T row holds this lane's 8 keys of k-step ks contiguously
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 v0 = *(const bf16x8 *)&sVb[ql * LROW + ks * 16 + hl * 8];
    const bf16x8 v1 = *(const bf16x8 *)&sVb[(32 + ql) * LROW + ks * 16 + hl * 8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      o[g][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pb[g][ks], o[g][0], 0, 0, 0);
      o[g][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pb[g][ks], o[g][1], 0, 0, 0);
    }
  }
}

template <int G>
__global__ __launch_bounds__(256) void attn_bf16_v2(AttnArgs a) {
  constexpr int QW = 32 * G, QB = 4 * QW;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][KV_T * LROW];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][64 * LROW];

  const int S = a.S_img + a.S_txt;
  int qb, h, b;
  attn_block_coords((S + QB - 1) / QB, a.H, qb, h, b);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q0 = qb * QB + wave * QW;
  const int64_t bh = (int64_t)b * a.H + h;
  const bf16 *Qg = (const bf16 *)a.Q + bh * a.S_pad * 64;
  const bf16 *Kg = (const bf16 *)a.K + bh * a.S_pad * 64;
  const bf16 *Vg = (const bf16 *)a.Vt + bh * 64 * a.S_pad;
  const int n_kv = kv_count(a, b);
  const int n_tiles = (n_kv + KV_T - 1) / KV_T;
  const int hl = lane >> 5, ql = lane & 31;

  bf16x8 qf[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int qr = q0 + g * 32 + ql;
    qr = qr < S ? qr : S - 1;
    const bf16 *src = Qg + (int64_t)qr * 64 + hl * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[g][ks] = *(const bf16x8 *)(src + ks * 16);
  }

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

  f32x16 o[G][2];
  float m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    o[g][0] = f32x16{};
    o[g][1] = f32x16{};
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
  }
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
    attn_tile<G, true>(sK[buf], sV[buf], qf, o, m_run, l_run, kv0, n_kv, ql, hl);
    if (more) {
      *(u32x4 *)&sK[buf ^ 1][l_off0] = rk0;
      *(u32x4 *)&sK[buf ^ 1][l_off1] = rk1;
      *(u32x4 *)&sV[buf ^ 1][l_off0] = rv0;
      *(u32x4 *)&sV[buf ^ 1][l_off1] = rv1;
    }
    __syncthreads();
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l_tot = l_run[g] + __shfl_xor(l_run[g], 32);
    const float inv = 1.0f / l_tot;
    const int p = q0 + g * 32 + ql;
    if (p >= S) continue;
    bf16 *dst = out_row<bf16>(a, b, p) + h * 64;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      bf16x4 v0, v1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] = (bf16)(o[g][0][gg * 4 + e] * inv);
        v1[e] = (bf16)(o[g][1][gg * 4 + e] * inv);
      }
      *(bf16x4 *)(dst + gg * 8 + hl * 4) = v0;
      *(bf16x4 *)(dst + 32 + gg * 8 + hl * 4) = v1;
    }
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
    hipLaunchKernelGGL(attn_bf16_v2<1>, dim3(((S + 127) / 128) * a.H * a.B), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_f32_simple, dim3((S + 63) / 64, a.H, a.B), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace lens

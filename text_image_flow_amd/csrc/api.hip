// C-ABI layer of the Lens denoiser library: argument checks, workspace
// carve-up and the launch sequences of one block, the whole denoiser and
// the flow step.  Host code only; every arithmetic step runs in the kernels.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/lens.h"
#include "common.h"

using namespace lens;

namespace {

thread_local std::string g_err;

lens_status fail(lens_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
lens_status fail(lens_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

// ------------------------------------------------------------ kernel timer
// Per calling thread: a thread that starts the timer records and reads only
// its own launches' events.  The events stay allocated for the thread's
// lifetime (reused by the next start).
struct Timer {
  uint32_t mask = 0;
  std::vector<hipEvent_t> pool;
  std::vector<int> kind_of;  // family of each recorded event pair
  std::vector<int> kernels;  // kernels launched inside each pair
  size_t used = 0;
};
thread_local Timer g_timer;

// Wraps one launch: records events around it when its family is timed.
struct Timed {
  bool on;
  hipStream_t st;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  Timed(lens_kernel_kind k, hipStream_t s) : on((g_timer.mask >> (int)k) & 1u), st(s) {
    if (!on) return;
    while (g_timer.pool.size() < g_timer.used + 2) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) {
        on = false;
        return;
      }
      g_timer.pool.push_back(e);
    }
    g_timer.kind_of.push_back((int)k);
    g_timer.kernels.push_back(1);
    e0 = g_timer.pool[g_timer.used++];
    e1 = g_timer.pool[g_timer.used++];
    (void)hipEventRecord(e0, st);
  }
  // `kernels`: how many kernels the timed call launched (one span of time)
  hipError_t done(hipError_t e, int kernels = 1) {
    if (on) {
      (void)hipEventRecord(e1, st);
      g_timer.kernels.back() = kernels;
    }
    return e;
  }
};

#define HIP_TRY(expr)                                                                           \
  do {                                                                                          \
    hipError_t _e = (expr);                                                                     \
    if (_e != hipSuccess) return fail(LENS_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------ checks
lens_status check_config(const lens_config *c) {
  if (!c) return fail(LENS_ERR_INVALID_ARG, "cfg is NULL");
  if (c->act_dtype != LENS_F32 && c->act_dtype != LENS_BF16)
    return fail(LENS_ERR_INVALID_ARG, "act_dtype %d is not LENS_F32 or LENS_BF16", (int)c->act_dtype);
  if (c->heads <= 0 || c->head_dim <= 0 || c->hidden != c->heads * c->head_dim)
    return fail(LENS_ERR_INVALID_ARG, "hidden (%d) must equal heads (%d) * head_dim (%d)", c->hidden, c->heads,
                c->head_dim);
  const int *ax = c->rope_axes;
  if (ax[0] < 0 || ax[1] < 0 || ax[2] < 0 || ax[0] % 2 || ax[1] % 2 || ax[2] % 2 ||
      ax[0] + ax[1] + ax[2] != c->head_dim)
    return fail(LENS_ERR_INVALID_ARG, "rope_axes (%d,%d,%d) must be even and sum to head_dim %d", ax[0], ax[1],
                ax[2], c->head_dim);
  if (c->head_dim != 64) return fail(LENS_ERR_UNSUPPORTED, "head_dim %d: only 64 is supported", c->head_dim);
  if (c->hidden % 256 || c->hidden > 2048)
    return fail(LENS_ERR_UNSUPPORTED, "hidden %d: must be a multiple of 256, at most 2048", c->hidden);
  if (c->mlp_hidden <= 0 || c->mlp_hidden % 128)
    return fail(LENS_ERR_UNSUPPORTED, "mlp_hidden %d: must be a positive multiple of 128", c->mlp_hidden);
  if (!(c->eps > 0.f) || !(c->rope_theta > 0.f))
    return fail(LENS_ERR_INVALID_ARG, "eps and rope_theta must be positive");
  if (c->gemm_fp8 != 0 && c->gemm_fp8 != 1) return fail(LENS_ERR_INVALID_ARG, "gemm_fp8 %d is not 0 or 1", c->gemm_fp8);
  if (c->gemm_fp8 && c->act_dtype != LENS_BF16)
    return fail(LENS_ERR_UNSUPPORTED, "gemm_fp8 requires act_dtype LENS_BF16");
  return LENS_OK;
}

lens_status check_dit_config(const lens_config *c) {
  lens_status s = check_config(c);
  if (s != LENS_OK) return s;
  if (c->n_blocks < 0) return fail(LENS_ERR_INVALID_ARG, "n_blocks %d < 0", c->n_blocks);
  if (c->in_ch <= 0 || c->in_ch % 64)
    return fail(LENS_ERR_UNSUPPORTED, "in_ch %d: must be a positive multiple of 64", c->in_ch);
  if (c->out_ch <= 0 || c->out_ch % 128)
    return fail(LENS_ERR_UNSUPPORTED, "out_ch %d: must be a positive multiple of 128", c->out_ch);
  if (c->txt_layers <= 0 || c->txt_feat_dim <= 0 || (c->txt_layers * c->txt_feat_dim) % 64)
    return fail(LENS_ERR_UNSUPPORTED, "txt_layers * txt_feat_dim must be a positive multiple of 64");
  if (c->t_freq_dim <= 0 || c->t_freq_dim % 16 || c->t_freq_dim > 2048)
    return fail(LENS_ERR_UNSUPPORTED, "t_freq_dim %d: must be a positive multiple of 16, at most 2048", c->t_freq_dim);
  return LENS_OK;
}

lens_status check_sizes(int B, int Si, int St) {
  if (B < 1 || Si < 1 || St < 0)
    return fail(LENS_ERR_INVALID_ARG, "need B >= 1, S_img >= 1, S_txt >= 0 (got %d, %d, %d)", B, Si, St);
  if ((int64_t)Si + St > (1 << 24)) return fail(LENS_ERR_UNSUPPORTED, "sequence too long");
  return LENS_OK;
}

// Device tensors that kernels read or write with 16-byte vector or buffer
// accesses (activations, weights, biases, scales, outputs) must start on a
// 16-byte boundary; NULL passes.
bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }

lens_status check_linear(const lens_linear &l, const char *name) {
  if (!l.w) return fail(LENS_ERR_INVALID_ARG, "weight %s is NULL", name);
  if (!al16(l.w) || !al16(l.b) || !al16(l.w_scale))
    return fail(LENS_ERR_INVALID_ARG, "weight %s: w, b and w_scale must be 16-byte aligned", name);
  return LENS_OK;
}

lens_status check_block_w(const lens_block_w *w, int idx, bool fp8) {
  if (!w) return fail(LENS_ERR_INVALID_ARG, "block %d weight table is NULL", idx);
  const lens_stream_w *s[2] = {&w->img, &w->txt};
  const char *nm[2] = {"img", "txt"};
  for (int i = 0; i < 2; ++i) {
    const lens_linear *ls[6] = {&s[i]->mod, &s[i]->qkv, &s[i]->out, &s[i]->w1, &s[i]->w3, &s[i]->w2};
    const char *ln[6] = {"mod", "qkv", "out", "w1", "w3", "w2"};
    for (int j = 0; j < 6; ++j) {
      if (!ls[j]->w) return fail(LENS_ERR_INVALID_ARG, "block %d %s.%s weight is NULL", idx, nm[i], ln[j]);
      if (fp8 && j > 0 && !ls[j]->w_scale)
        return fail(LENS_ERR_INVALID_ARG, "block %d %s.%s: gemm_fp8 needs w_scale", idx, nm[i], ln[j]);
      if (!al16(ls[j]->w) || !al16(ls[j]->b) || !al16(ls[j]->w_scale))
        return fail(LENS_ERR_INVALID_ARG, "block %d %s.%s: w, b and w_scale must be 16-byte aligned", idx, nm[i],
                    ln[j]);
    }
    if (!s[i]->q_gain || !s[i]->k_gain)
      return fail(LENS_ERR_INVALID_ARG, "block %d %s q/k gain is NULL", idx, nm[i]);
    if (!al16(s[i]->q_gain) || !al16(s[i]->k_gain))
      return fail(LENS_ERR_INVALID_ARG, "block %d %s q/k gains must be 16-byte aligned", idx, nm[i]);
  }
  return LENS_OK;
}

// ------------------------------------------------------------ workspace
struct BlockWs {
  float *mod;                 // [2][B][6D]
  void *a_img, *a_txt;        // [B*S, D] act: norm output, then attention output
  void *qkv_img, *qkv_txt;    // [B*S, 3D] act; reused for the SwiGLU output [B*S, mlp]
  void *Q, *K, *V;            // joint layout [B, H, S_pad, 64]
  float2 *rope;               // bf16 path: [S_img + S_txt][32] (cos, sin)
  // gemm_fp8: the projections' inputs as MX fp8 (e4m3 rows, E8M0 scales
  // [rows, K / 32]): q8/s8 [B*S, hidden] from the norms and the attention,
  // f8/fs8 [B*S, mlp_hidden] from the SwiGLU epilogue
  void *q8_img, *q8_txt, *s8_img, *s8_txt;
  void *f8_img, *f8_txt, *fs8_img, *fs8_txt;
  size_t bytes;
};

int s_pad(int Si, int St) { return ((Si + St + 63) / 64) * 64; }

BlockWs carve_block(const lens_config *c, int B, int Si, int St, char *base, bool with_mod) {
  const size_t es = c->act_dtype == LENS_BF16 ? 2 : 4;
  const size_t D = c->hidden;
  const size_t wide = 3 * D > (size_t)c->mlp_hidden ? 3 * D : (size_t)c->mlp_hidden;
  const size_t Sp = s_pad(Si, St);
  BlockWs w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    void *p = base ? base + off : nullptr;
    off += align_up(n);
    return p;
  };
  w.mod = with_mod ? (float *)take(2 * (size_t)B * 6 * D * 4) : nullptr;
  w.a_img = take((size_t)B * Si * D * es);
  w.a_txt = take((size_t)B * St * D * es);
  w.qkv_img = take((size_t)B * Si * wide * es);
  w.qkv_txt = take((size_t)B * St * wide * es);
  w.Q = take((size_t)B * c->heads * Sp * 64 * es);
  w.K = take((size_t)B * c->heads * Sp * 64 * es);
  w.V = take((size_t)B * c->heads * Sp * 64 * es);
  w.rope = (float2 *)take((size_t)(Si + St) * 32 * sizeof(float2));
  if (c->gemm_fp8) {
    const size_t F = (size_t)c->mlp_hidden;
    w.q8_img = take((size_t)B * Si * D);
    w.q8_txt = take((size_t)B * St * D);
    w.s8_img = take((size_t)B * Si * D / 32);
    w.s8_txt = take((size_t)B * St * D / 32);
    w.f8_img = take((size_t)B * Si * F);
    w.f8_txt = take((size_t)B * St * F);
    w.fs8_img = take((size_t)B * Si * F / 32);
    w.fs8_txt = take((size_t)B * St * F / 32);
  }
  w.bytes = off;
  return w;
}

struct DitWs {
  float *phi, *h1, *temb, *mods, *nmod;
  float *h_img, *h_txt;
  void *tn;
  BlockWs blk;
  size_t bytes;
};

DitWs carve_dit(const lens_config *c, int B, int Si, int St, char *base) {
  const size_t es = c->act_dtype == LENS_BF16 ? 2 : 4;
  const size_t D = c->hidden;
  DitWs w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    void *p = base ? base + off : nullptr;
    off += align_up(n);
    return p;
  };
  w.phi = (float *)take((size_t)B * c->t_freq_dim * 4);
  w.h1 = (float *)take((size_t)B * D * 4);
  w.temb = (float *)take((size_t)B * D * 4);
  w.mods = (float *)take((size_t)c->n_blocks * 2 * B * 6 * D * 4);
  w.nmod = (float *)take((size_t)B * 2 * D * 4);
  w.h_img = (float *)take((size_t)B * Si * D * 4);
  w.h_txt = (float *)take((size_t)B * St * D * 4);
  w.tn = take((size_t)B * St * c->txt_layers * c->txt_feat_dim * es);
  w.blk = carve_block(c, B, Si, St, base ? base + off : nullptr, false);
  off += w.blk.bytes;
  w.bytes = off;
  return w;
}

// ------------------------------------------------------------ launches
lens_status gemm(lens_kernel_kind, int epi, bool bf, GemmProblem *p, int np, hipStream_t st) {
  Timed t(LENS_KERNEL_GEMM, st);
  const hipError_t r = launch_gemm(epi, bf, p, np, st);
  hipError_t e = t.done(r, gemm_kernels_launched());
  if (e != hipSuccess) return fail(LENS_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e));
  return LENS_OK;
}

// Point both problems of a grouped projection at MX fp8 inputs (x8/xs8 of
// the image and text rows) and the layers' fp8 weights.
void to_fp8(GemmProblem *g, const lens_linear &li, const lens_linear &lt, const lens_linear *l3i,
            const lens_linear *l3t, void *x8_img, void *xs8_img, void *x8_txt, void *xs8_txt) {
  g[0].A = x8_img;
  g[0].A_scale = xs8_img;
  g[0].W_scale = li.w_scale;
  g[0].W3_scale = l3i ? l3i->w_scale : nullptr;
  g[1].A = x8_txt;
  g[1].A_scale = xs8_txt;
  g[1].W_scale = lt.w_scale;
  g[1].W3_scale = l3t ? l3t->w_scale : nullptr;
}

lens_status gemm8(int epi, GemmProblem *p, hipStream_t st, const QkvOut *qo = nullptr) {
  Timed t(LENS_KERNEL_GEMM, st);
  const hipError_t r = launch_gemm_fp8(epi, p, 2, st, qo);
  hipError_t e = t.done(r, gemm_kernels_launched());
  if (e != hipSuccess) return fail(LENS_ERR_HIP, "fp8 GEMM launch failed: %s", hipGetErrorString(e));
  return LENS_OK;
}

#define LTRY(expr)                   \
  do {                               \
    lens_status _s = (expr);         \
    if (_s != LENS_OK) return _s;    \
  } while (0)

// bf16 path, once per forward call: the RoPE table of the joint sequence
// (shared by every block) and zeroed padding rows of Q, K, V (the QKV
// epilogue writes valid rows only; V rows beyond the last key must be finite).
lens_status prepare_joint(const lens_config *c, const int32_t *img_pos, const int32_t *txt_pos, int B, int Si, int St,
                          const BlockWs &ws, hipStream_t st) {
  if (c->act_dtype != LENS_BF16) return LENS_OK;
  Timed t(LENS_KERNEL_QKNORM_ROPE, st);
  hipError_t e = launch_rope_table(img_pos, txt_pos, Si, St, c->rope_axes[0], c->rope_axes[1], c->rope_axes[2],
                                   c->rope_theta, ws.rope, st);
  if (e == hipSuccess) e = launch_zero_pad_rows(ws.Q, ws.K, ws.V, B, c->heads, Si + St, s_pad(Si, St), st);
  e = t.done(e);
  if (e != hipSuccess) return fail(LENS_ERR_HIP, "RoPE table / padding launch failed: %s", hipGetErrorString(e));
  return LENS_OK;
}

// The block after AdaLN: mod_img / mod_txt point at [B][6D] rows.
lens_status block_core(const lens_config *c, const lens_block_w *w, float *h_img, float *h_txt, const float *mod_img,
                       const float *mod_txt, const int32_t *img_pos, const int32_t *txt_pos, const int32_t *txt_len,
                       int B, int Si, int St, const BlockWs &ws, hipStream_t st) {
  const bool bf = c->act_dtype == LENS_BF16;
  const int D = c->hidden, D6 = 6 * D;
  const int Mi = B * Si, Mt = B * St;
  hipError_t e;

  // gemm_fp8: every projection input is produced as MX fp8 by the kernel
  // before it (norms, attention, SwiGLU epilogue), never stored as bf16
  const bool f8 = c->gemm_fp8 != 0;
  // 1. pre-attention RMSNorm + modulation (shift1, scale1)
  NormModProblem nm[2] = {
      {h_img, f8 ? ws.q8_img : ws.a_img, mod_img, mod_img + D, D6, Mi, Si > 0 ? Si : 1, ws.s8_img},
      {h_txt, f8 ? ws.q8_txt : ws.a_txt, mod_txt, mod_txt + D, D6, Mt, St > 0 ? St : 1, ws.s8_txt}};
  {
    Timed t(LENS_KERNEL_NORM, st);
    e = t.done(launch_norm_modulate(nm, 2, D, c->eps, bf, st, f8));
    if (e != hipSuccess) return fail(LENS_ERR_HIP, "norm launch failed: %s", hipGetErrorString(e));
  }
  // 2. QKV projections, 3. QK RMSNorm + RoPE -> joint Q, K, V.  bf16: one
  // GEMM whose epilogue normalises, rotates and scatters the heads (the
  // RoPE table and zeroed padding rows come from prepare_joint); fp32:
  // GEMM into qkv, then the separate QK-norm/RoPE kernel.
  GemmProblem g[2] = {};
  g[0] = GemmProblem{ws.a_img, w->img.qkv.w, nullptr, w->img.qkv.b, nullptr, ws.qkv_img, nullptr, 0, 1, Mi, 3 * D, D};
  g[1] = GemmProblem{ws.a_txt, w->txt.qkv.w, nullptr, w->txt.qkv.b, nullptr, ws.qkv_txt, nullptr, 0, 1, Mt, 3 * D, D};
  const int Sp = s_pad(Si, St);
  if (bf) {
    QkvOut qo{ws.Q, ws.K, ws.V, {w->img.q_gain, w->txt.q_gain}, {w->img.k_gain, w->txt.k_gain}, ws.rope,
              Si, St, Sp, c->heads, c->eps, 0.125f * 1.4426950408889634f};   // attention takes Q in log2 units
    if (f8) {
      to_fp8(g, w->img.qkv, w->txt.qkv, nullptr, nullptr, ws.q8_img, ws.s8_img, ws.q8_txt, ws.s8_txt);
      LTRY(gemm8(EPI_QKV, g, st, &qo));
    } else {
      Timed t(LENS_KERNEL_GEMM, st);
      e = launch_gemm(EPI_QKV, true, g, 2, st, &qo);
      e = t.done(e, gemm_kernels_launched());
      if (e != hipSuccess) return fail(LENS_ERR_HIP, "QKV GEMM launch failed: %s", hipGetErrorString(e));
    }
  } else {
    LTRY(gemm(LENS_KERNEL_GEMM, EPI_STORE, bf, g, 2, st));
    QkRopeArgs qa{ws.qkv_img, ws.qkv_txt, w->img.q_gain, w->img.k_gain, w->txt.q_gain, w->txt.k_gain, img_pos,
                  txt_pos, ws.Q, ws.K, ws.V, B, c->heads, Si, St, Sp, c->rope_axes[0], c->rope_axes[1],
                  c->rope_axes[2], c->rope_theta, c->eps, 1.0f};
    Timed t(LENS_KERNEL_QKNORM_ROPE, st);
    e = t.done(launch_qknorm_rope(qa, false, st));
    if (e != hipSuccess) return fail(LENS_ERR_HIP, "qk-norm/rope launch failed: %s", hipGetErrorString(e));
  }
  // 4. joint attention; outputs overwrite the (dead) norm outputs
  AttnArgs aa{ws.Q, ws.K, ws.V, ws.a_img, ws.a_txt, txt_len, B, c->heads, Si, St, Sp, 0.125f,
              {w->img.q_gain, w->img.k_gain, w->txt.q_gain, w->txt.k_gain}};
  if (f8) {
    aa.O8_img = ws.q8_img;
    aa.O8_txt = ws.q8_txt;
    aa.OS_img = ws.s8_img;
    aa.OS_txt = ws.s8_txt;
  }
  {
    Timed t(LENS_KERNEL_ATTENTION, st);
    e = t.done(launch_attention(aa, bf, st));
    if (e != hipSuccess) return fail(LENS_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  }
  // 5. output projection + gated residual (gate1)
  g[0] = GemmProblem{ws.a_img, w->img.out.w, nullptr, w->img.out.b, nullptr, h_img, mod_img + 2 * D, D6, Si > 0 ? Si : 1,
                     Mi, D, D};
  g[1] = GemmProblem{ws.a_txt, w->txt.out.w, nullptr, w->txt.out.b, nullptr, h_txt, mod_txt + 2 * D, D6, St > 0 ? St : 1,
                     Mt, D, D};
  if (f8) {
    to_fp8(g, w->img.out, w->txt.out, nullptr, nullptr, ws.q8_img, ws.s8_img, ws.q8_txt, ws.s8_txt);
    LTRY(gemm8(EPI_GATED, g, st));
  } else {
    LTRY(gemm(LENS_KERNEL_GEMM, EPI_GATED, bf, g, 2, st));
  }
  // 6. pre-MLP RMSNorm + modulation (shift2, scale2)
  nm[0].shift = mod_img + 3 * D;
  nm[0].scale = mod_img + 4 * D;
  nm[1].shift = mod_txt + 3 * D;
  nm[1].scale = mod_txt + 4 * D;
  {
    Timed t(LENS_KERNEL_NORM, st);
    e = t.done(launch_norm_modulate(nm, 2, D, c->eps, bf, st, f8));
    if (e != hipSuccess) return fail(LENS_ERR_HIP, "norm launch failed: %s", hipGetErrorString(e));
  }
  // 7. w1 | w3 with the SwiGLU epilogue (output reuses the qkv buffers)
  const int F = c->mlp_hidden;
  g[0] = GemmProblem{ws.a_img, w->img.w1.w, w->img.w3.w, w->img.w1.b, w->img.w3.b, ws.qkv_img, nullptr, 0, 1, Mi, F, D};
  g[1] = GemmProblem{ws.a_txt, w->txt.w1.w, w->txt.w3.w, w->txt.w1.b, w->txt.w3.b, ws.qkv_txt, nullptr, 0, 1, Mt, F, D};
  if (f8) {
    to_fp8(g, w->img.w1, w->txt.w1, &w->img.w3, &w->txt.w3, ws.q8_img, ws.s8_img, ws.q8_txt, ws.s8_txt);
    g[0].C = ws.f8_img;
    g[0].C_scale = ws.fs8_img;
    g[1].C = ws.f8_txt;
    g[1].C_scale = ws.fs8_txt;
    LTRY(gemm8(EPI_SWIGLU_MX, g, st));
  } else {
    LTRY(gemm(LENS_KERNEL_GEMM, EPI_SWIGLU, bf, g, 2, st));
  }
  // 8. w2 + gated residual (gate2)
  g[0] = GemmProblem{ws.qkv_img, w->img.w2.w, nullptr, w->img.w2.b, nullptr, h_img, mod_img + 5 * D, D6, Si > 0 ? Si : 1,
                     Mi, D, F};
  g[1] = GemmProblem{ws.qkv_txt, w->txt.w2.w, nullptr, w->txt.w2.b, nullptr, h_txt, mod_txt + 5 * D, D6, St > 0 ? St : 1,
                     Mt, D, F};
  if (f8) {
    to_fp8(g, w->img.w2, w->txt.w2, nullptr, nullptr, ws.f8_img, ws.fs8_img, ws.f8_txt, ws.fs8_txt);
    LTRY(gemm8(EPI_GATED, g, st));
  } else {
    LTRY(gemm(LENS_KERNEL_GEMM, EPI_GATED, bf, g, 2, st));
  }
  return LENS_OK;
}

// AdaLN modulation of `nblk` blocks from SiLU(temb), plus, when extra is not
// NULL, one more GEMV of the same input (the final layer's modulation, N =
// extra_n, into extra_y).  mods: [nblk][2][B][6D].  The problems go out in
// as few launches of at most GEMV_MAX_PROBS as there can be, split evenly.
lens_status adaln_all(const lens_config *c, const lens_block_w *const *blocks, int nblk, const float *temb, int B,
                      float *mods, hipStream_t st, const lens_linear *extra = nullptr, float *extra_y = nullptr,
                      int extra_n = 0) {
  const bool bf = c->act_dtype == LENS_BF16;
  const int D = c->hidden, D6 = 6 * D;
  const int total = 2 * nblk + (extra ? 1 : 0);
  const int launches = (total + GEMV_MAX_PROBS - 1) / GEMV_MAX_PROBS;
  GemvBatch gb{};
  int done = 0, launched = 0;
  auto flush = [&]() -> lens_status {
    if (gb.nprob == 0) return LENS_OK;
    Timed t(LENS_KERNEL_ADALN, st);
    hipError_t e = t.done(launch_gemv(gb, temb, B, D, true, bf, st));
    done += gb.nprob;
    ++launched;
    gb.nprob = 0;
    if (e != hipSuccess) return fail(LENS_ERR_HIP, "AdaLN launch failed: %s", hipGetErrorString(e));
    return LENS_OK;
  };
  // problems of the current launch: an even share of what is left
  auto share = [&]() { return (total - done + (launches - launched) - 1) / (launches - launched); };
  auto add = [&](const void *w, const void *b, float *y, int n) -> lens_status {
    const int k = gb.nprob++;
    gb.W[k] = w;
    gb.bias[k] = b;
    gb.y[k] = y;
    gb.N[k] = n;
    gb.y_stride[k] = n;
    return gb.nprob == share() ? flush() : LENS_OK;
  };
  for (int i = 0; i < nblk; ++i) {
    for (int s = 0; s < 2; ++s) {
      const lens_linear &l = s == 0 ? blocks[i]->img.mod : blocks[i]->txt.mod;
      LTRY(add(l.w, l.b, mods + ((size_t)i * 2 + s) * B * D6, D6));
    }
  }
  if (extra) LTRY(add(extra->w, extra->b, extra_y, extra_n));
  return flush();
}

}  // namespace

// ====================================================================== ABI
extern "C" {

void lens_default_config(lens_config *c, int32_t act) {
  if (!c) return;
  c->hidden = 1536;
  c->heads = 24;
  c->head_dim = 64;
  c->mlp_hidden = 4096;
  c->n_blocks = 48;
  c->rope_axes[0] = 8;
  c->rope_axes[1] = 28;
  c->rope_axes[2] = 28;
  c->in_ch = 128;
  c->out_ch = 128;
  c->txt_feat_dim = 2880;
  c->txt_layers = 4;
  c->t_freq_dim = 256;
  c->rope_theta = 10000.f;
  c->eps = 1e-6f;
  c->t_scale = 1000.f;
  c->act_dtype = act;
  c->gemm_fp8 = 0;
}

size_t lens_block_workspace_bytes(const lens_config *c, int32_t B, int32_t Si, int32_t St) {
  if (check_config(c) != LENS_OK || check_sizes(B, Si, St) != LENS_OK) return 0;
  return carve_block(c, B, Si, St, nullptr, true).bytes;
}

size_t lens_dit_workspace_bytes(const lens_config *c, int32_t B, int32_t Si, int32_t St) {
  if (check_dit_config(c) != LENS_OK || check_sizes(B, Si, St) != LENS_OK) return 0;
  return carve_dit(c, B, Si, St, nullptr).bytes;
}

lens_status lens_block_forward(const lens_config *c, const lens_block_w *w, float *h_img, float *h_txt,
                               const float *temb, const int32_t *img_pos, const int32_t *txt_pos,
                               const int32_t *txt_len, int32_t B, int32_t Si, int32_t St, void *workspace,
                               size_t ws_bytes, void *hip_stream) {
  LTRY(check_config(c));
  LTRY(check_sizes(B, Si, St));
  LTRY(check_block_w(w, 0, c->gemm_fp8));
  if (!h_img || !temb || !img_pos) return fail(LENS_ERR_INVALID_ARG, "h_img, temb and img_pos must not be NULL");
  if (St > 0 && (!h_txt || !txt_pos)) return fail(LENS_ERR_INVALID_ARG, "h_txt and txt_pos must not be NULL");
  if (!al16(h_img) || !al16(h_txt)) return fail(LENS_ERR_INVALID_ARG, "h_img and h_txt must be 16-byte aligned");
  const BlockWs need = carve_block(c, B, Si, St, nullptr, true);
  if (!workspace || ws_bytes < need.bytes)
    return fail(LENS_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace ? ws_bytes : 0, need.bytes);
  if ((uintptr_t)workspace % 256) return fail(LENS_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t st = (hipStream_t)hip_stream;
  const BlockWs ws = carve_block(c, B, Si, St, (char *)workspace, true);
  const lens_block_w *bl[1] = {w};
  LTRY(adaln_all(c, bl, 1, temb, B, ws.mod, st));
  const float *mod_img = ws.mod, *mod_txt = ws.mod + (size_t)B * 6 * c->hidden;
  LTRY(prepare_joint(c, img_pos, txt_pos, B, Si, St, ws, st));
  return block_core(c, w, h_img, h_txt, mod_img, mod_txt, img_pos, txt_pos, txt_len, B, Si, St, ws, st);
}

}  // extern "C"

namespace {

// Arguments of the whole-denoiser call, checked before any device work.
lens_status check_dit_call(const lens_config *c, const lens_dit_w *w, const void *x, const void *txt_feats,
                           const float *t, const int32_t *img_pos, const int32_t *txt_pos, int32_t B, int32_t Si,
                           int32_t St, const float *v_out) {
  LTRY(check_dit_config(c));
  LTRY(check_sizes(B, Si, St));
  if (!w) return fail(LENS_ERR_INVALID_ARG, "weight table is NULL");
  LTRY(check_linear(w->t_fc1, "t_fc1"));
  LTRY(check_linear(w->t_fc2, "t_fc2"));
  LTRY(check_linear(w->img_in, "img_in"));
  LTRY(check_linear(w->txt_in, "txt_in"));
  LTRY(check_linear(w->norm_out, "norm_out"));
  LTRY(check_linear(w->proj_out, "proj_out"));
  if (!w->txt_gain) return fail(LENS_ERR_INVALID_ARG, "txt_gain is NULL");
  if (!al16(w->txt_gain)) return fail(LENS_ERR_INVALID_ARG, "txt_gain must be 16-byte aligned");
  if (c->n_blocks > 0 && !w->blocks) return fail(LENS_ERR_INVALID_ARG, "blocks is NULL");
  for (int i = 0; i < c->n_blocks; ++i) LTRY(check_block_w(&w->blocks[i], i, c->gemm_fp8));
  if (!x || !t || !img_pos || !v_out) return fail(LENS_ERR_INVALID_ARG, "x, t, img_pos and v_out must not be NULL");
  if (St > 0 && (!txt_feats || !txt_pos))
    return fail(LENS_ERR_INVALID_ARG, "txt_feats and txt_pos must not be NULL");
  if (!al16(x) || !al16(txt_feats) || !al16(v_out))
    return fail(LENS_ERR_INVALID_ARG, "x, txt_feats and v_out must be 16-byte aligned");
  return LENS_OK;
}

// The whole denoiser on a checked call, with its scratch at `base` (256-byte
// aligned, carve_dit(...).bytes long).
lens_status dit_run(const lens_config *c, const lens_dit_w *w, const void *x, const void *txt_feats, const float *t,
                    const int32_t *img_pos, const int32_t *txt_pos, const int32_t *txt_len, int32_t B, int32_t Si,
                    int32_t St, float *v_out, char *base, hipStream_t st) {
  const bool bf = c->act_dtype == LENS_BF16;
  const DitWs ws = carve_dit(c, B, Si, St, base);
  const int D = c->hidden;
  hipError_t e;
  // timestep embedding: phi(t) -> fc1 -> SiLU -> fc2
  HIP_TRY(launch_timestep_features(t, ws.phi, B, c->t_freq_dim, c->t_scale, st));
  {
    GemvBatch gb{};
    gb.nprob = 1;
    gb.W[0] = w->t_fc1.w;
    gb.bias[0] = w->t_fc1.b;
    gb.y[0] = ws.h1;
    gb.N[0] = D;
    gb.y_stride[0] = D;
    Timed tt(LENS_KERNEL_ADALN, st);
    e = tt.done(launch_gemv(gb, ws.phi, B, c->t_freq_dim, false, bf, st));
    if (e != hipSuccess) return fail(LENS_ERR_HIP, "timestep fc1 failed: %s", hipGetErrorString(e));
    gb.W[0] = w->t_fc2.w;
    gb.bias[0] = w->t_fc2.b;
    gb.y[0] = ws.temb;
    Timed t2(LENS_KERNEL_ADALN, st);
    e = t2.done(launch_gemv(gb, ws.h1, B, D, true, bf, st));
    if (e != hipSuccess) return fail(LENS_ERR_HIP, "timestep fc2 failed: %s", hipGetErrorString(e));
  }
  // AdaLN of every block (temb does not depend on the block) + norm_out
  {
    std::vector<const lens_block_w *> bl(c->n_blocks);
    for (int i = 0; i < c->n_blocks; ++i) bl[i] = &w->blocks[i];
    LTRY(adaln_all(c, bl.data(), c->n_blocks, ws.temb, B, ws.mods, st, &w->norm_out, ws.nmod, 2 * D));
  }
  // embeddings
  GemmProblem g{x, w->img_in.w, nullptr, w->img_in.b, nullptr, ws.h_img, nullptr, 0, 1, B * Si, D, c->in_ch};
  LTRY(gemm(LENS_KERNEL_GEMM, EPI_STORE_F32, bf, &g, 1, st));
  if (St > 0) {
    HIP_TRY(launch_txt_norm(txt_feats, w->txt_gain, ws.tn, B * St, c->txt_layers, c->txt_feat_dim, c->eps, bf, st));
    g = GemmProblem{ws.tn, w->txt_in.w, nullptr, w->txt_in.b, nullptr, ws.h_txt, nullptr, 0, 1, B * St, D,
                    c->txt_layers * c->txt_feat_dim};
    LTRY(gemm(LENS_KERNEL_GEMM, EPI_STORE_F32, bf, &g, 1, st));
  }
  // blocks
  LTRY(prepare_joint(c, img_pos, txt_pos, B, Si, St, ws.blk, st));
  for (int i = 0; i < c->n_blocks; ++i) {
    const float *mi = ws.mods + (size_t)i * 2 * B * 6 * D;
    const float *mt = mi + (size_t)B * 6 * D;
    LTRY(block_core(c, &w->blocks[i], ws.h_img, ws.h_txt, mi, mt, img_pos, txt_pos, txt_len, B, Si, St, ws.blk, st));
  }
  // final layer
  NormModProblem nm[1] = {{ws.h_img, ws.blk.a_img, ws.nmod, ws.nmod + D, 2 * D, B * Si, Si}};
  {
    Timed tt(LENS_KERNEL_NORM, st);
    e = tt.done(launch_norm_modulate(nm, 1, D, c->eps, bf, st));
    if (e != hipSuccess) return fail(LENS_ERR_HIP, "norm_out launch failed: %s", hipGetErrorString(e));
  }
  g = GemmProblem{ws.blk.a_img, w->proj_out.w, nullptr, w->proj_out.b, nullptr, v_out, nullptr, 0, 1, B * Si,
                  c->out_ch, D};
  LTRY(gemm(LENS_KERNEL_GEMM, EPI_STORE_F32, bf, &g, 1, st));
  return LENS_OK;
}

// File-scope device scratch of lens_dit_forward_noalloc.  Every device the
// library runs on holds its own copy from the load of this code object until
// the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in there).
static __device__ __align__(256) unsigned char scratch[LENS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of the current device's scratch, looked up once per device.
lens_status static_scratch(void **out) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LENS_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LENS_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LENS_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return LENS_OK;
}

}  // namespace

extern "C" {

lens_status lens_dit_forward(const lens_config *c, const lens_dit_w *w, const void *x, const void *txt_feats,
                             const float *t, const int32_t *img_pos, const int32_t *txt_pos, const int32_t *txt_len,
                             int32_t B, int32_t Si, int32_t St, float *v_out, void *workspace, size_t ws_bytes,
                             void *hip_stream) {
  LTRY(check_dit_call(c, w, x, txt_feats, t, img_pos, txt_pos, B, Si, St, v_out));
  const DitWs need = carve_dit(c, B, Si, St, nullptr);
  if (!workspace || ws_bytes < need.bytes)
    return fail(LENS_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace ? ws_bytes : 0, need.bytes);
  if ((uintptr_t)workspace % 256) return fail(LENS_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return dit_run(c, w, x, txt_feats, t, img_pos, txt_pos, txt_len, B, Si, St, v_out, (char *)workspace,
                 (hipStream_t)hip_stream);
}

lens_status lens_dit_forward_noalloc(const lens_config *c, const lens_dit_w *w, const void *x, const void *txt_feats,
                                     const float *t, const int32_t *img_pos, const int32_t *txt_pos,
                                     const int32_t *txt_len, int32_t B, int32_t Si, int32_t St, float *v_out,
                                     void *hip_stream) {
  LTRY(check_dit_call(c, w, x, txt_feats, t, img_pos, txt_pos, B, Si, St, v_out));
  const DitWs need = carve_dit(c, B, Si, St, nullptr);
  if (need.bytes > LENS_NOALLOC_SCRATCH_BYTES)
    return fail(LENS_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu",
                need.bytes, (size_t)LENS_NOALLOC_SCRATCH_BYTES);
  void *base = nullptr;
  LTRY(static_scratch(&base));
  return dit_run(c, w, x, txt_feats, t, img_pos, txt_pos, txt_len, B, Si, St, v_out, (char *)base,
                 (hipStream_t)hip_stream);
}

lens_status lens_flow_step(float *x, const float *v_cond, const float *v_uncond, int64_t n, float dt,
                           float cfg_scale, void *x_lowp_out, int32_t lowp_dtype, void *hip_stream) {
  if (n < 0) return fail(LENS_ERR_INVALID_ARG, "n = %lld < 0", (long long)n);
  if (n > 0 && (!x || !v_cond)) return fail(LENS_ERR_INVALID_ARG, "x and v_cond must not be NULL");
  if (x_lowp_out && lowp_dtype != LENS_F32 && lowp_dtype != LENS_BF16)
    return fail(LENS_ERR_INVALID_ARG, "lowp_dtype %d is not LENS_F32 or LENS_BF16", (int)lowp_dtype);
  HIP_TRY(launch_flow_step(x, v_cond, v_uncond, n, dt, cfg_scale, x_lowp_out, lowp_dtype == LENS_BF16,
                           (hipStream_t)hip_stream));
  return LENS_OK;
}

lens_status lens_flow_step_rescaled(float *x, const float *v_cond, const float *v_uncond, int64_t n_tokens,
                                    int32_t channels, float dt, float cfg_scale, void *x_lowp_out,
                                    int32_t lowp_dtype, void *hip_stream) {
  if (n_tokens < 0) return fail(LENS_ERR_INVALID_ARG, "n_tokens = %lld < 0", (long long)n_tokens);
  if (channels <= 0) return fail(LENS_ERR_INVALID_ARG, "channels = %d must be positive", (int)channels);
  if (n_tokens > 0 && (!x || !v_cond)) return fail(LENS_ERR_INVALID_ARG, "x and v_cond must not be NULL");
  if (x_lowp_out && lowp_dtype != LENS_F32 && lowp_dtype != LENS_BF16)
    return fail(LENS_ERR_INVALID_ARG, "lowp_dtype %d is not LENS_F32 or LENS_BF16", (int)lowp_dtype);
  if (n_tokens > ((int64_t)1 << 40) / channels) return fail(LENS_ERR_UNSUPPORTED, "too many elements");
  HIP_TRY(launch_flow_step_rescaled(x, v_cond, v_uncond, n_tokens, channels, dt, cfg_scale, x_lowp_out,
                                    lowp_dtype == LENS_BF16, (hipStream_t)hip_stream));
  return LENS_OK;
}

lens_status lens_quantize_mxfp8(const void *src, int32_t src_dtype, int64_t rows, int32_t cols,
                                int32_t scale_layout, void *q_out, void *scale_out, void *hip_stream) {
  if (src_dtype != LENS_F32 && src_dtype != LENS_BF16)
    return fail(LENS_ERR_INVALID_ARG, "src_dtype %d is not LENS_F32 or LENS_BF16", (int)src_dtype);
  if (scale_layout != LENS_MX_ROWS && scale_layout != LENS_MX_SLABS)
    return fail(LENS_ERR_INVALID_ARG, "scale_layout %d is not LENS_MX_ROWS or LENS_MX_SLABS", (int)scale_layout);
  const int unit = scale_layout == LENS_MX_SLABS ? 128 : 32;
  if (rows < 0 || cols <= 0 || cols % unit)
    return fail(LENS_ERR_INVALID_ARG, "rows %lld / cols %d: need rows >= 0 and cols a positive multiple of %d",
                (long long)rows, (int)cols, unit);
  if (rows > 0 && (!src || !q_out || !scale_out)) return fail(LENS_ERR_INVALID_ARG, "NULL pointer");
  if (!al16(src) || !al16(q_out)) return fail(LENS_ERR_INVALID_ARG, "src and q_out must be 16-byte aligned");
  if (rows > (((int64_t)1 << 40) / cols)) return fail(LENS_ERR_UNSUPPORTED, "too many elements");
  MxQuantProblem q{src, q_out, scale_out, rows};
  HIP_TRY(launch_mx_quant(&q, 1, cols, src_dtype == LENS_BF16, scale_layout == LENS_MX_SLABS,
                          (hipStream_t)hip_stream));
  return LENS_OK;
}

lens_status lens_timer_start(uint32_t mask) {
  if (mask >> LENS_KERNEL_COUNT) return fail(LENS_ERR_INVALID_ARG, "kernel mask 0x%x has unknown bits", mask);
  g_timer.mask = mask;
  g_timer.used = 0;
  g_timer.kind_of.clear();
  g_timer.kernels.clear();
  return LENS_OK;
}

lens_status lens_timer_stop(double *ms, int64_t *launches) {
  double acc[LENS_KERNEL_COUNT] = {0};
  int64_t cnt[LENS_KERNEL_COUNT] = {0};
  const size_t n = g_timer.used / 2;
  g_timer.mask = 0;
  g_timer.used = 0;
  for (size_t i = 0; i < n; ++i) {
    HIP_TRY(hipEventSynchronize(g_timer.pool[2 * i + 1]));
    float f = 0.f;
    HIP_TRY(hipEventElapsedTime(&f, g_timer.pool[2 * i], g_timer.pool[2 * i + 1]));
    acc[g_timer.kind_of[i]] += f;
    cnt[g_timer.kind_of[i]] += g_timer.kernels[i];
  }
  g_timer.kind_of.clear();
  g_timer.kernels.clear();
  for (int k = 0; k < LENS_KERNEL_COUNT; ++k) {
    if (ms) ms[k] = acc[k];
    if (launches) launches[k] = cnt[k];
  }
  return LENS_OK;
}

lens_status lens_time_grid(int32_t steps, float mu, int32_t has_mu, float *t_out, float *dt_out) {
  if (steps < 1) return fail(LENS_ERR_INVALID_ARG, "steps = %d: need at least one step", (int)steps);
  if (has_mu && !std::isfinite(mu)) return fail(LENS_ERR_INVALID_ARG, "mu is not finite");
  // t_k = 1 - k / steps, optionally moved by mu in logit space:
  // t' = e^mu t / (e^mu t + 1 - t), which keeps 0 and 1 fixed
  const double e = has_mu ? std::exp((double)mu) : 1.0;
  auto point = [&](int k) {
    const double t = 1.0 - (double)k / steps;
    return has_mu ? e * t / (e * t + 1.0 - t) : t;
  };
  for (int k = 0; k <= steps; ++k) {
    const double t = point(k);
    if (t_out) t_out[k] = (float)t;
    if (dt_out && k < steps) dt_out[k] = (float)(point(k + 1) - t);
  }
  return LENS_OK;
}

lens_status lens_mu_for_tokens(int64_t n_tokens, double n0, double mu0, double n1, double mu1, double *mu_out) {
  if (!mu_out) return fail(LENS_ERR_INVALID_ARG, "mu_out is NULL");
  if (!std::isfinite(n0) || !std::isfinite(n1) || !std::isfinite(mu0) || !std::isfinite(mu1))
    return fail(LENS_ERR_INVALID_ARG, "line points must be finite");
  if (n0 == n1) return fail(LENS_ERR_INVALID_ARG, "the line needs two distinct token counts (n0 == n1 = %g)", n0);
  *mu_out = mu0 + ((double)n_tokens - n0) * (mu1 - mu0) / (n1 - n0);
  return LENS_OK;
}

const char *lens_status_string(int32_t s) {
  switch (s) {
    case LENS_OK: return "LENS_OK";
    case LENS_ERR_INVALID_ARG: return "LENS_ERR_INVALID_ARG";
    case LENS_ERR_UNSUPPORTED: return "LENS_ERR_UNSUPPORTED";
    case LENS_ERR_WORKSPACE: return "LENS_ERR_WORKSPACE";
    case LENS_ERR_HIP: return "LENS_ERR_HIP";
  }
  return "unknown lens_status";
}

const char *lens_last_error(void) { return g_err.c_str(); }

const char *lens_version(void) { return "lens-mi355x 0.1 (gfx950)"; }

}  // extern "C"

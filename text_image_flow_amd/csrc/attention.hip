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
//   * a wave owns 32 queries; four waves share 64-key K and V tiles that
//     direct global->LDS loads double-buffer in LDS;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: each lane then holds one
//     query (lane & 31) and 32 of the tile's 64 keys, so the row max needs
//     one exchange with the partner lane (lane ^ 32) and the row sum none
//     until the end;
//   * P^T is rounded to bf16 in registers and used directly as the B operand
//     of O^T += V^T P^T; V stays row-major ([S_pad, 64], like K) and
//     ds_read_b64_tr_b16 assembles the transposed operand from it; O^T keeps
//     one query per lane, so the online-softmax rescale is a per-lane scalar;
//   * Q arrives pre-scaled by scale * log2(e), and the QK MFMAs start from
//     -m, so p = exp2(s) with no subtraction; the running max is lazy and
//     row sums add the fp32 probabilities with plain adds (the PV product
//     takes them rounded to bf16);
//   * the grid is flat and XCD-aware (one head's q-blocks share an L2);
//   * O is written as bf16 rows, or (MX fp8 projections) as e4m3 rows with
//     one E8M0 scale per 32 dims, quantized from fp32 in registers.
// fp32 path: one thread per query, plain loops (correctness only).
#include "common.h"

namespace lens {

namespace {

constexpr int KV_T = 64;        // keys per tile

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

// Lazy running max: rows rescale only when a tile's max exceeds the running
// max by more than TAU (log2 units), so probabilities stay <= 2^TAU.
constexpr float TAU = 8.0f;
// largest score bound used as a fixed max: p >= 2^(-2 BOUND_MAX) keeps
// probabilities and row sums far above fp32 / bf16 underflow
constexpr float BOUND_MAX = 48.0f;

// -------------------------------------------------------------- bf16
// K and V tiles arrive by direct global->LDS loads (raw buffer loads with
// the lds bit: one wave instruction fills 1 KB = 8 rows of 128 bytes) into
// a double-buffered ring, so no VGPRs stage them; each lane keeps a
// constant 32-bit offset inside the (sample, head) slice and the tile's
// offset rides in the scalar offset, so a tile's loads need no vector
// address arithmetic.  Rows are unpadded; 16-byte chunk c of row r sits in slot
// c ^ ((r >> 1) & 7): the 16 lanes that one LDS cycle serves read 16
// consecutive rows, and these land on 16 distinct 16-byte bank groups of the
// 64 banks (a plain c ^ (r & 7) maps rows r and r + 8 onto the same group).
// The partial last tile is peeled so the steady-state loop carries no mask.
typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from base + voff + soff into LDS at M0 + 16 * lane
// (bounds: bytes)
__device__ __forceinline__ void buffer_lds16(const void *base, int bytes, lds_void_t *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, bytes, 0x00020000),
                                           dst, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8)); }
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// V tiles are row-major [key][64 dims] like K tiles, 16-byte chunk c of
// key row r in slot c ^ vswz(r).  The PV MFMA wants V^T fragments (row =
// dim, k = keys), which ds_read_tr16_b64 assembles: within each 16-lane
// group, lane j reads 4 consecutive dims of key j / 4 and lane i gets back
// dim i of those 4 keys.  The 8 keys a lane feeds per k-step follow the
// P^T operand's k-slot order (slot s holds key s with bits 2 and 3
// swapped): keys 4 hl .. 4 hl + 3 and 8 + 4 hl .. 8 + 4 hl + 3.  vswz puts
// the 4 key rows one 16-lane read touches on 8 distinct bank groups.
__device__ __forceinline__ int vswz(int r) { return ((r >> 1) & 1) * 4; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// byte offset inside a V tile of lane's first transpose read for k-step 0,
// dim half 0 (vlane), and the fragment for (ks, dh)
__device__ __forceinline__ int v_lane_row(int lane) { return 4 * (lane >> 5) + ((lane & 15) >> 2); }
__device__ __forceinline__ int v_lane_dim(int lane) { return ((lane >> 4) & 1) * 16 + 4 * (lane & 3); }
__device__ __forceinline__ bf16x8 v_frag(const char *sVb, int ks, int dh, int lane) {
  const int dim = dh * 32 + v_lane_dim(lane);
  bf16x8 v;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int key = ks * 16 + 8 * r + v_lane_row(lane);
    const int off = key * 128 + (((dim >> 3) ^ vswz(key)) << 4) + (dim & 7) * 2;
    const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)((__attribute__((address_space(3))) char *)sVb + off));
    const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * r + e] = tb[e];
  }
  return v;
}

// One 64-key tile.  FIRST: the S accumulators start at 0, the tile's max
// becomes the running max m and p = exp2(s - m).  Otherwise they start at
// minit = -m (16 copies), so the MFMAs deliver s - m directly and p = exp2(.)
// needs no subtraction; only when a tile's max exceeds m by more than TAU
// is m raised (O and l rescaled, this tile's values shifted).
//   BOUNDED: every score is known to be <= m = -minit[0] (a bound from the
//   q/k gains, see attn_bf16), so the max tracking and rescaling are skipped;
//   the QK MFMAs start from -m on every tile.
template <bool FIRST, bool MASK, bool BOUNDED>
__device__ __forceinline__ void attn_tile(const char *sKb, const char *sVb, const bf16x8 (&qf)[4], f32x16 (&o)[2],
                                             float &m_run, float &l_run, f32x16 &minit, int kv0, int n_kv, int ql,
                                             int hl) {
  const int vlane = hl * 32 + ql;
  const int sw = (ql >> 1) & 7;   // rows ql and 32 + ql share the swizzle
  // keys 0-31 (s0) fully before keys 32-63 (s1), so that in the bounded
  // case the exponentials of s0 can go out while the s1 MFMAs still run
  f32x16 s0, s1;
  {
    const f32x16 c0 = (FIRST && !BOUNDED) ? f32x16{} : minit;
    s0 = c0;
    s1 = c0;
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int slot = ((ks * 2 + hl) ^ sw) << 4;
    const bf16x8 k0 = *(const bf16x8 *)(sKb + ql * 128 + slot);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], s0, 0, 0, 0);
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int slot = ((ks * 2 + hl) ^ sw) << 4;
    const bf16x8 k1 = *(const bf16x8 *)(sKb + (32 + ql) * 128 + slot);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[ks], s1, 0, 0, 0);
  }
  if constexpr (MASK) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = kv0 + (r >> 2) * 8 + hl * 4 + (r & 3);
      if (kv >= n_kv) s0[r] = -INFINITY;
      if (kv + 32 >= n_kv) s1[r] = -INFINITY;
    }
  }
  if constexpr (!BOUNDED) {
  float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if constexpr (FIRST) {
    m_run = mx;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] -= mx;
      s1[r] -= mx;
      minit[r] = -mx;
    }
  } else {
    if (__any(mx > TAU)) {
      // raise the running max by this tile's excess (per lane, >= 0)
      const float d = fmaxf(mx, 0.f);
      const float alpha = __builtin_amdgcn_exp2f(-d);
      m_run += d;
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[0][r] *= alpha;
        o[1][r] *= alpha;
        s0[r] -= d;
        s1[r] -= d;
        minit[r] = -m_run;
      }
    }
  }
  }
  // probabilities of keys 0-31 (P^T k steps 0, 1), their PV MFMAs, then
  // keys 32-63 (k steps 2, 3).  The PV product takes them rounded to bf16;
  // the row sum adds their fp32 values with plain adds, which issue
  // alongside another wave's MFMAs (measured on MI355X: v_add_f32 from a
  // second wave of the SIMD overlaps MFMA work fully, v_dot2_f32_bf16 not at
  // all).  One add chain: a second one costs the registers that keep three
  // waves per SIMD.
  bf16x8 pb[4];
  float lsum = l_run;   // the row sum continues the running sum directly
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const f32x16 &sh = half ? s1 : s0;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float x0 = __builtin_amdgcn_exp2f(sh[e]), x1 = __builtin_amdgcn_exp2f(sh[e + 1]);
      const float x2 = __builtin_amdgcn_exp2f(sh[8 + e]), x3 = __builtin_amdgcn_exp2f(sh[9 + e]);
      bf16x2 p0 = {(bf16)x0, (bf16)x1};
      bf16x2 p1 = {(bf16)x2, (bf16)x3};
      lsum += x0;
      lsum += x1;
      lsum += x2;
      lsum += x3;
      pb[2 * half][e] = p0[0]; pb[2 * half][e + 1] = p0[1];
      pb[2 * half + 1][e] = p1[0]; pb[2 * half + 1][e + 1] = p1[1];
    }
#pragma unroll
    for (int ks = 2 * half; ks < 2 * half + 2; ++ks) {
      const bf16x8 v0 = v_frag(sVb, ks, 0, vlane);
      const bf16x8 v1 = v_frag(sVb, ks, 1, vlane);
      o[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pb[ks], o[0], 0, 0, 0);
      o[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pb[ks], o[1], 0, 0, 0);
    }
  }
  l_run = lsum;
}

// three waves per SIMD (168 VGPRs) are what the tile loop is scheduled for
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_bf16(AttnArgs a) {
  constexpr int TILE_BYTES = 64 * 128;        // K tile or V tile (row-major)
  constexpr int STAGE = 2 * TILE_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int S = a.S_img + a.S_txt;
  int qb, h, b;
  attn_block_coords((S + 127) / 128, a.H, qb, h, b);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = qb * 128 + wave * 32;
  const int64_t bh = (int64_t)b * a.H + h;
  const bf16 *Qg = (const bf16 *)a.Q + bh * a.S_pad * 64;
  const bf16 *Kg = (const bf16 *)a.K + bh * a.S_pad * 64;
  const bf16 *Vg = (const bf16 *)a.V + bh * a.S_pad * 64;
  const int n_kv = kv_count(a, b);
  // a q-block holding only padded text queries (the sample's valid tokens,
  // image and text, are its first n_kv): their rows are unspecified, so
  // none of the block's work is needed
  if (qb * 128 >= n_kv) return;
  const int n_tiles = (n_kv + KV_T - 1) / KV_T;
  const int n_full = n_kv / KV_T;
  const int hl = lane >> 5, ql = lane & 31;

  bf16x8 qf[4];
  {
    int qr = q0 + ql;
    qr = qr < S ? qr : S - 1;
    const bf16 *src = Qg + (int64_t)qr * 64 + hl * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *(const bf16x8 *)(src + ks * 16);
  }
  // each wave fills rows [wave * 16, wave * 16 + 16) of the K and V tiles:
  // two instructions of 8 rows each; lane -> row + lane / 8, slot lane % 8
  const int r0 = wave * 16 + (lane >> 3), r1 = r0 + 8, slot = lane & 7;
  const int k_off0 = r0 * 128 + ((slot ^ ((r0 >> 1) & 7)) * 16);
  const int k_off1 = r1 * 128 + ((slot ^ ((r1 >> 1) & 7)) * 16);
  const int v_off0 = r0 * 128 + ((slot ^ vswz(r0)) * 16);
  const int v_off1 = r1 * 128 + ((slot ^ vswz(r1)) * 16);
  const int slice_bytes = a.S_pad * 128;      // one (sample, head) slice of K or V
  const int dst0 = wave * 16 * 128, dst1 = dst0 + 8 * 128;
#define ATT_ISSUE(t_, stage_)                                                                               \
  do {                                                                                                      \
    char *sb_ = smem + (stage_) * STAGE;                                                                    \
    const int so_ = (t_) * KV_T * 128;                                                                      \
    buffer_lds16(Kg, slice_bytes, (lds_void_t *)(sb_ + dst0), k_off0, so_);                                \
    buffer_lds16(Kg, slice_bytes, (lds_void_t *)(sb_ + dst1), k_off1, so_);                                \
    buffer_lds16(Vg, slice_bytes, (lds_void_t *)(sb_ + TILE_BYTES + dst0), v_off0, so_);                   \
    buffer_lds16(Vg, slice_bytes, (lds_void_t *)(sb_ + TILE_BYTES + dst1), v_off1, so_);                   \
  } while (0)

  // Score bound: q and k are RMS-normalised per head (norm < 8 before the
  // gain), scaled by at most max|gain|, rotated (norm kept) and q is scaled
  // by log2(e) / 8, so |s| <= 8 log2(e) max|g_q| max|g_k| over both
  // streams' gains; the margin covers the bf16 rounding of q and k.  With
  // the bound as the subtracted max, p = exp2(s - m) needs no running max
  // (softmax does not depend on the constant) as long as 2^(-2m) stays far
  // from fp32 underflow, i.e. m <= BOUND_MAX; otherwise the online max runs.
  float m_bound = INFINITY;
  if (a.gain[0] && a.gain[1] && a.gain[2] && a.gain[3]) {
    const float gq = fmaxf(fabsf((float)((const bf16 *)a.gain[0])[lane]), fabsf((float)((const bf16 *)a.gain[2])[lane]));
    const float gk = fmaxf(fabsf((float)((const bf16 *)a.gain[1])[lane]), fabsf((float)((const bf16 *)a.gain[3])[lane]));
    float mq = gq, mk = gk;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) {
      mq = fmaxf(mq, __shfl_xor(mq, sh));
      mk = fmaxf(mk, __shfl_xor(mk, sh));
    }
    m_bound = __uint_as_float(
        __builtin_amdgcn_readfirstlane(__float_as_uint(8.0f * 1.4426950408889634f * mq * mk * 1.02f + 0.02f)));
  }

  f32x16 o[2] = {f32x16{}, f32x16{}};
  f32x16 minit;
  float m_run = 0.f, l_run = 0.f;
  ATT_ISSUE(0, 0);
  // tile 0 (always holds image keys, so at least one valid key per row)
  wait_vmcnt0();
  __builtin_amdgcn_s_barrier();
  if (1 < n_tiles) ATT_ISSUE(1, 1);
// one full tile t held in stage st_ (= t & 1): wait for this wave's part of
// it, and for its own reads of tile t - 1, then the barrier frees stage
// 1 - st_ for tile t + 1
#define ATT_STEP(t_, st_, BND)                                                                              \
  do {                                                                                                      \
    wait_vmcnt0();                                                                                          \
    wait_lgkmcnt0();                                                                                        \
    __builtin_amdgcn_s_barrier();                                                                           \
    if ((t_) + 1 < n_tiles) ATT_ISSUE((t_) + 1, 1 - (st_));                                                 \
    const char *sb_ = smem + (st_) * STAGE;                                                                 \
    attn_tile<false, false, BND>(sb_, sb_ + TILE_BYTES, qf, o, m_run, l_run, minit, (t_) * KV_T, n_kv, ql, hl); \
  } while (0)
#define ATT_TILES(BND)                                                                                      \
  do {                                                                                                      \
    if (n_full >= 1)                                                                                        \
      attn_tile<true, false, BND>(smem, smem + TILE_BYTES, qf, o, m_run, l_run, minit, 0, n_kv, ql, hl);    \
    else                                                                                                    \
      attn_tile<true, true, BND>(smem, smem + TILE_BYTES, qf, o, m_run, l_run, minit, 0, n_kv, ql, hl);     \
    /* two tiles per trip: odd tiles sit in stage 1, even ones in stage 0, */                               \
    /* so every LDS address is a fixed offset from a loop-invariant base */                                 \
    int t = 1;                                                                                              \
    for (; t + 1 < n_full; t += 2) {                                                                        \
      ATT_STEP(t, 1, BND);                                                                                  \
      ATT_STEP(t + 1, 0, BND);                                                                              \
    }                                                                                                       \
    if (t < n_full) ATT_STEP(t, 1, BND);                                                                    \
    if (n_full < n_tiles && n_full >= 1) {                                                                  \
      wait_vmcnt0();                                                                                        \
      wait_lgkmcnt0();                                                                                      \
      __builtin_amdgcn_s_barrier();                                                                         \
      const char *sb = smem + (n_full & 1) * STAGE;                                                         \
      attn_tile<false, true, BND>(sb, sb + TILE_BYTES, qf, o, m_run, l_run, minit, n_full * KV_T, n_kv, ql,  \
                                  hl);                                                                      \
    }                                                                                                       \
  } while (0)
  if (m_bound <= BOUND_MAX) {
#pragma unroll
    for (int r = 0; r < 16; ++r) minit[r] = -m_bound;
    ATT_TILES(true);
  } else {
    ATT_TILES(false);
  }
#undef ATT_TILES
#undef ATT_STEP
#undef ATT_ISSUE

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  const int p = q0 + ql;
  if (p >= S) return;   // lanes l and l ^ 32 share p: pairs stay whole
  if (a.O8_img) {
    // MX fp8 output: the head's dims 0-31 (o[0]) and 32-63 (o[1]) are one
    // block each, 16 values on this lane (dims 8 gg + 4 hl + e) and 16 on
    // lane l ^ 32; after the swaps lanes 0-31 hold bytes 0-15 of a block
    // and lanes 32-63 bytes 16-31
    const int D = a.H * 64;
    const bool img = p < a.S_img;
    const int64_t row = img ? (int64_t)b * a.S_img + p : (int64_t)b * a.S_txt + (p - a.S_img);
    unsigned char *q8 = (unsigned char *)(img ? a.O8_img : a.O8_txt) + row * D + h * 64;
    unsigned char *sc = (unsigned char *)(img ? a.OS_img : a.OS_txt);
    const int64_t srows = (int64_t)a.B * (img ? a.S_img : a.S_txt);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float am = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) am = fmaxf(am, fabsf(o[t][k] * inv));
      const auto sa = __builtin_amdgcn_permlane32_swap(__float_as_uint(am), __float_as_uint(am), false, false);
      const int ex = mx_exponent(fmaxf(__uint_as_float(sa[0]), __uint_as_float(sa[1])));
      unsigned d[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        d[gg] = mx_pack4(o[t][gg * 4] * inv, o[t][gg * 4 + 1] * inv, o[t][gg * 4 + 2] * inv, o[t][gg * 4 + 3] * inv,
                         ex);
      const auto s0 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
      *(u32x4 *)(q8 + t * 32 + 16 * hl) = u32x4{s0[0], s0[1], s1[0], s1[1]};
      if (hl == 0) sc[mx_scale_index(row, h * 2 + t, srows)] = (unsigned char)(ex + 127);
    }
    return;
  }
  bf16 *dst = out_row<bf16>(a, b, p) + h * 64;
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    bf16x4 v0, v1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v0[e] = (bf16)(o[0][gg * 4 + e] * inv);
      v1[e] = (bf16)(o[1][gg * 4 + e] * inv);
    }
    *(bf16x4 *)(dst + gg * 8 + hl * 4) = v0;
    *(bf16x4 *)(dst + 32 + gg * 8 + hl * 4) = v1;
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
  const float *Vg = (const float *)a.V + bh * a.S_pad * 64;
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
      sV[d][r] = Vg[(int64_t)(kv0 + r) * 64 + d];
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
    hipLaunchKernelGGL(attn_bf16, dim3(((S + 127) / 128) * a.H * a.B), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_f32_simple, dim3((S + 63) / 64, a.H, a.B), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace lens

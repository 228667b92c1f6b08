// Dynamic split-KV paged decode attention for MI355X (gfx950 / CDNA4).
//
// Two launches per decode step.  Workgroup (w, h) handles the work items that
// the host plan gives workgroup w, for kv head h (grid = W * Hkv, kv head
// fastest).  Each workgroup is 4 waves; the waves of a workgroup take the
// 32-token chunks of an item round-robin, keep their own online-softmax
// state, and combine through LDS when the item ends.  An item that covers a
// whole request writes its output; the other items write a normalised
// partial and its log-sum-exp, which a second, small kernel merges per
// request in slot order.
//
// Method: page "Tencent HPC llega a SGLang y desafía a los kernels de
// inferencia predeterminados" (remio.ai), section "Por qué Tencent HPC
// importa para el serving de modelos en línea" -- KV work cut into uniform
// tiles and spread over thread blocks by the current lengths; arex-research
// page, Dynamic Attention paragraphs -- a persistent kernel allocating tiles
// per decode step by actual KV length; "vLLM × HPC-Ops" summary page -- the
// load-balanced scheduler replaces fixed split-KV scheduling and a fused
// RoPE + QK-Norm + KV-write prologue precedes attention.  The exact merge of
// split partials by log-sum-exp and the online softmax are the standard
// exact form of split-KV attention; the page layout, tile shapes and MFMA
// mapping below are this library's own.
//
// Data path per chunk (32 tokens, one wave): K and V rows come straight from
// HBM into VGPRs through buffer loads whose resource covers only the valid
// rows of the page (rows past len read as zero, so poisoned or stale rows are
// never seen).  QK^T and PV run on v_mfma_f32_16x16x32_bf16 with the group of
// q heads padded to 16; V is transposed in registers (16-bit lane-local
// shuffles) to give the PV product its token-contiguous operand.  The path is
// HBM-bound (8 flop per KV byte for bf16), so MFMA only does the small dense
// products.
#include <hip/hip_runtime.h>
#include <float.h>
#include <algorithm>
#include <mutex>
#include <type_traits>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "hda.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWaves = 4;             // waves per workgroup
constexpr int kChunk = 32;            // tokens per wave per step
constexpr int kMaxGroup = 16;         // q heads per kv head (MFMA N)
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource dword 3 for gfx9 raw buffers

struct Args {
  const uint16_t* q;
  uint8_t* k_pages;
  uint8_t* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* plan;
  float* out;
  float* part_o;
  float* part_lse;
  uint16_t* q_prime;     // workspace copy of the prologue's q' (bf16 [B][Hq][D])
  int32_t* req_slots;    // device-planned launches: per request (first slot, slot count)
  int32_t* check;        // per tile workgroup: HDA_CHECK_* bits of this call (null: none)
  int32_t* cover;        // coverage launches: visits per (page, row, kv head)
  const int32_t* rows;   // multi-token launches: row blocks [n][4] (request, first packed
                         // row, rows, position of the first row)
  const uint16_t* q_norm_w;
  const uint16_t* k_norm_w;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const float* k_scales;   // per-head [Hkv] or per-page [num_pages][Hkv] factors
  const float* v_scales;
  int64_t page_stride;   // bytes per page (all kv heads)
  int32_t num_pages;     // page ids are int32; clamped on the host
  int32_t head_stride;   // bytes per (page, kv head) slab
  int32_t batch, n_q_heads, n_kv_heads, group;
  int32_t page_size, log2_ps, max_pages;
  int32_t n_wg, n_items, n_parts;
  int32_t tile_len;      // device-planned launches only
  int32_t qb;            // query rows per block: partial slots hold qb x Hq rows (1 for decode)
  int32_t n_req;         // requests (block-table rows); multi-token launches
  int32_t scale_mode;    // HDA_SCALE_*
  int32_t v_dim_major;   // V pages [page][Hkv][D][page_size] instead of [..][page_size][D]
  float qk_scale_log2;   // sm_scale * k_scale * log2(e)
  float v_scale;
  float k_scale, rms_eps, rope_theta;
};

template <int D, bool FP8>
struct Geo {
  static constexpr int ELEM = FP8 ? 1 : 2;
  static constexpr int RB = D * ELEM;        // bytes per token row of one head
  static constexpr int KL = D * ELEM / 64;   // 16-byte K loads per lane per 16-token half
  static constexpr int VW = D * ELEM / 64;   // dwords of V per token per lane
  static constexpr int DPL = D / 16;         // output d values per lane (PV N blocks)
  static constexpr int STEPS = D / 32;       // QK k-steps of 32
  // register sets in the per-wave chunk ring (a third set for fp8 pushed the
  // kernel past 256 VGPRs into spills and measured slower)
  static constexpr int NBUF = 2;
};

// Registers of one in-flight chunk (ks, vs: the K and V scale factors of the
// page under each 16-token half; used with per-page scales only).
template <int D, bool FP8>
struct Chunk {
  u32x4 k[2][Geo<D, FP8>::KL];
  uint32_t v[8][Geo<D, FP8>::VW];
  float ks[2], vs[2];
};

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes,
                                           kRsrcWord3);
}

__device__ inline float bf16_bits_to_float(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Four OCP E4M3FN codes -> four bf16 (exact: every code is a bf16 value).
// gfx950's scaled pair conversion with scale 1.0 writes two bf16 per
// instruction; it agrees with the exact decode on all 256 codes.
__device__ inline void fp8x4_to_bf16x4(uint32_t c, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true));
}

// fp32 -> OCP E4M3FN code: round to nearest, ties to even, saturating at
// +-448, NaN -> 0x7F.  Written from the format: subnormals are multiples of
// 2^-9 below 2^-6; a normal binade [2^e, 2^(e+1)) holds 8 steps of 2^(e-3).
__device__ inline uint32_t fp8_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a == a)) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);
  int e;
  (void)frexpf(a, &e);                      // a = m * 2^e, m in [0.5, 1)
  const float q = rintf(ldexpf(a, 4 - e));  // 1.mmm scaled to [8, 16]
  uint32_t code = (uint32_t)((e + 6) << 3) + ((uint32_t)q - 8u);  // q == 16 carries
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Rotary angles: inverse frequency theta^(-2l/D) for lane l < D/2 in double
// precision (computed once per wave), the angle pos * inv_freq in double,
// reduced to [-pi, pi] in double, then cos/sin in float.  The reduction keeps
// the float rounding of the angle at ~1e-7 rad for positions up to 2^31.
__device__ inline double rope_inv_freq(int lane, int D, float theta) {
  return exp(-(2.0 * (double)lane / (double)D) * log((double)theta));
}

__device__ inline void rope_cos_sin(int pos, double inv_freq, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double phi = (double)pos * inv_freq;
  const double r = phi - rint(phi * inv_two_pi) * two_pi;
  sincosf((float)r, &s, &c);
}

// RMSNorm (over D, weight w) then rotate-half RoPE of one head vector held as
// (x0 = x[lane], x1 = x[lane + D/2]) on lanes < D/2.
__device__ inline void norm_rope(float& x0, float& x1, bool act, const uint16_t* w, int lane,
                                 int D, float eps, float c, float s) {
  const float ss = wave_sum(act ? x0 * x0 + x1 * x1 : 0.0f);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  if (act) {
    const float y0 = x0 * r * bf16_bits_to_float(w[lane]);
    const float y1 = x1 * r * bf16_bits_to_float(w[lane + D / 2]);
    x0 = y0 * c - y1 * s;
    x1 = y1 * c + y0 * s;
  }
}

// Start of the 8 contiguous head dims a lane feeds to QK step s.  Any
// assignment works as long as K and q use the same one; this one makes each
// lane's K load 16 contiguous bytes.
template <bool FP8>
__device__ inline int qk_dim(int s, int kg) {
  return FP8 ? 64 * (s >> 1) + 16 * kg + 8 * (s & 1) : 32 * s + 8 * kg;
}

template <int D, bool FP8>
__device__ inline bf16x8 k_operand(const Chunk<D, FP8>& ch, int hf, int s) {
  if constexpr (!FP8) {
    return __builtin_bit_cast(bf16x8, ch.k[hf][s]);
  } else {
    const u32x4 raw = ch.k[hf][s >> 1];
    const uint32_t c0 = (s & 1) ? raw[2] : raw[0];
    const uint32_t c1 = (s & 1) ? raw[3] : raw[1];
    uint32_t o0, o1, o2, o3;
    fp8x4_to_bf16x4(c0, o0, o1);
    fp8x4_to_bf16x4(c1, o2, o3);
    return __builtin_bit_cast(bf16x8, u32x4{o0, o1, o2, o3});
  }
}

// Buffer resources for the two 16-token halves of chunk c of (request b,
// kv head h).  A half with no valid rows (past len, outside the block table
// or an out-of-range page id) gets an empty resource and reads zeros.
// With PAGE, also the page's K and V scale factors of each half (1 for a
// half without rows, whose tokens are masked).  They are vector loads that
// nothing reads until the chunk is computed, so their wait is the one the
// chunk's own K/V loads need anyway (consuming them here would stall on
// every load in flight).
template <int D, bool FP8, bool PAGE>
__device__ inline void chunk_rsrc(const Args& a, const int32_t* __restrict__ block_table, int b,
                                  int L, int h, int c, bool live,
                                  __amdgpu_buffer_rsrc_t (&kr)[2],
                                  __amdgpu_buffer_rsrc_t (&vr)[2], Chunk<D, FP8>& ch) {
  using G = Geo<D, FP8>;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int t = c * kChunk + 16 * hf;
    int rows = L - t;
    rows = rows > 16 ? 16 : rows;
    int64_t off = 0;
    int bytes = 0;
    float ks = 1.f, vs = 1.f;
    if (live && rows > 0) {
      const int pidx = t >> a.log2_ps;
      if (pidx < a.max_pages) {
        const int page = block_table[(int64_t)b * a.max_pages + pidx];
        if (page >= 0 && page < a.num_pages) {
          off = (int64_t)page * a.page_stride + (int64_t)h * a.head_stride +
                (int64_t)(t & (a.page_size - 1)) * G::RB;
          bytes = rows * G::RB;
          if constexpr (PAGE) {
            const int64_t si = (int64_t)page * a.n_kv_heads + h;
            ks = a.k_scales[si];
            vs = a.v_scales[si];
          }
        }
      }
    }
    kr[hf] = make_rsrc(a.k_pages + off, bytes);
    vr[hf] = make_rsrc(a.v_pages + off, bytes);
    if constexpr (PAGE) {
      ch.ks[hf] = ks;
      ch.vs[hf] = vs;
    }
  }
}

// K/V rows are read once per step and never again by this launch: load them
// non-temporally (cache policy aux = nt) so they do not displace anything.
constexpr int kStreamAux = 2;

template <int D, bool FP8>
__device__ inline void issue_chunk(Chunk<D, FP8>& ch, const __amdgpu_buffer_rsrc_t (&kr)[2],
                                   const __amdgpu_buffer_rsrc_t (&vr)[2], int i, int kg) {
  using G = Geo<D, FP8>;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int u = 0; u < G::KL; ++u)
      ch.k[hf][u] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr[hf], i * G::RB + 64 * u + 16 * kg, 0, kStreamAux));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int hf = j >> 2;
    const int off = (4 * kg + (j & 3)) * G::RB + i * G::VW * 4;
    if constexpr (G::VW == 4) {
      const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr[hf], off, 0, kStreamAux));
      ch.v[j][0] = x[0]; ch.v[j][1] = x[1]; ch.v[j][2] = x[2]; ch.v[j][3] = x[3];
    } else if constexpr (G::VW == 2) {
      const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(vr[hf], off, 0, kStreamAux));
      ch.v[j][0] = x[0]; ch.v[j][1] = x[1];
    } else {
      ch.v[j][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(vr[hf], off, 0, kStreamAux);
    }
  }
}

// Max and sum over the four lanes (i, kg = 0..3) that share a column i:
// gfx950's lane swaps exchange the 16-lane rows 0<->1, 2<->3 (xor 16) and
// the 32-lane halves (xor 32) without going through LDS.
__device__ inline float kg_reduce_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float kg_reduce_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Maximum of two scores (numbers or -inf) as v_med3_f32(a, b, +inf), with
// +inf in a register the compiler does not see through (it would turn the
// median back into fmaxf, which on matrix-core results costs a NaN-quieting
// maximum per operand).
__device__ inline float opaque_inf() {
  float x = INFINITY;
  asm("" : "+v"(x));
  return x;
}
__device__ inline float qmax(float a, float b, float inf) {
  return __builtin_amdgcn_fmed3f(a, b, inf);
}
__device__ inline float kg_reduce_qmax(float x, float inf) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = qmax(__uint_as_float(a[0]), __uint_as_float(a[1]), inf);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return qmax(__uint_as_float(b[0]), __uint_as_float(b[1]), inf);
}

// Online-softmax update for one 32-token chunk of scores sacc (MFMA C
// layout: lane (i = lane % 16, kg = lane / 16) holds the scores of column i
// for tokens 16*hf + 4*kg + r in sacc[hf][r]): scale, mask, new running max,
// rescale of l and of the PV accumulators, and the bf16 weights for the PV
// product (k index 8*kg + j <-> token 16*(j/4) + 4*kg + j%4).
//
// With PAGE, the scores of each half take its page's K factor ks[hf], and
// the PV weights its page's V factor vs[hf]: the MFMA gets bf16(p * vs), and
// the running sum adds that rounded weight divided by vs, so the normaliser
// counts exactly the weight each V row received.
//
// With PF (multi-token rows), column i also stops at its own causal limit
// lim (lim_min: the smallest over the columns, wave-uniform), and a column
// whose tokens are all masked so far keeps m = -inf without producing NaN.
//
// The PV accumulators hold column i in lane (i, kg) (the score layout), so
// the rescale by alpha needs no exchange between lanes.  (The decode path,
// compute_chunk, keeps its own copy of these steps for its accumulator
// layout, column 4*kg + r in acc[nb][r].)
template <int DPL, bool PAGE, bool PF>
__device__ __attribute__((always_inline)) inline bf16x8 softmax_update(const f32x4 (&sacc)[2], const float (&ks)[2],
                                        const float (&vs)[2], int c, int k0, int k1, int lim,
                                        int lim_min, float qk_scale_log2, int kg, float& m_run,
                                        float& l_run, f32x4 (&acc)[DPL]) {
  float qs[2] = {qk_scale_log2, qk_scale_log2};
  if constexpr (PAGE) {
    qs[0] *= ks[0];
    qs[1] *= ks[1];
  }
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sc[j] = sacc[j >> 2][j & 3] * qs[j >> 2];
  const int t0 = c * kChunk;
  // partial chunk: mask tokens outside [k0, k1) (and, for PF, past lim)
  if (t0 < k0 || t0 + kChunk > k1 || (PF && t0 + kChunk - 1 > lim_min)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + 16 * (j >> 2) + 4 * kg + (j & 3);
      if (t < k0 || t >= k1 || (PF && t > lim)) sc[j] = -INFINITY;
    }
  }
  float mx = sc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
  mx = kg_reduce_max(mx);
  const float m_max = fmaxf(m_run, mx);
  // a column with every token masked so far: subtract 0, so that its weights
  // and alpha come out 0 (not NaN) and its state stays empty
  const float m_new = (PF && m_max == -INFINITY) ? 0.f : m_max;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  bf16x8 pop;
  float psum = 0.f;
  if constexpr (!PAGE) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 p = (__bf16)__builtin_amdgcn_exp2f(sc[j] - m_new);
      pop[j] = p;
      psum += (float)p;   // normalise with the same rounded weights PV uses
    }
  } else {
    const float rvs[2] = {__builtin_amdgcn_rcpf(vs[0]), __builtin_amdgcn_rcpf(vs[1])};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 p = (__bf16)(__builtin_amdgcn_exp2f(sc[j] - m_new) * vs[j >> 2]);
      pop[j] = p;
      psum += (float)p * rvs[j >> 2];
    }
  }
  l_run = l_run * alpha + psum;
  m_run = m_max;
  if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
    for (int nb = 0; nb < DPL; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nb][r] *= alpha;
  }
  return pop;
}

// One chunk: S^T = K Q^T on MFMA, online-softmax update, acc += P V on MFMA.
// Lane (i = lane % 16, kg = lane / 16): score of q head i for tokens
// 16*hf + 4*kg + r; PV accumulator for q head 4*kg + r, head dim DPL*i + nb.
//
// With PAGE, the scores of each half take its page's K factor, and the PV
// weights its page's V factor: the MFMA gets bf16(p * vs), and the running
// sum adds that rounded weight divided by vs, so the normaliser counts
// exactly the weight each V row received.
//
// With PF (multi-token rows), column i also stops at its own causal limit
// lim (lim_min: the smallest over the columns, wave-uniform), and a column
// whose tokens are all masked so far keeps m = -inf without producing NaN.
template <int D, bool FP8, bool PAGE, bool PF>
__device__ inline void compute_chunk(const Chunk<D, FP8>& ch, const bf16x8 (&qop)[Geo<D, FP8>::STEPS],
                                     int c, int k0, int k1, int lim, int lim_min,
                                     float qk_scale_log2, int kg, float& m_run, float& l_run,
                                     f32x4 (&acc)[Geo<D, FP8>::DPL]) {
  using G = Geo<D, FP8>;
  f32x4 sacc[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    sacc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < G::STEPS; ++s)
      sacc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<D, FP8>(ch, hf, s), qop[s],
                                                         sacc[hf], 0, 0, 0);
  }
  float qs[2] = {qk_scale_log2, qk_scale_log2};
  if constexpr (PAGE) {
    qs[0] *= ch.ks[0];
    qs[1] *= ch.ks[1];
  }
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sc[j] = sacc[j >> 2][j & 3] * qs[j >> 2];
  const int t0 = c * kChunk;
  // partial chunk: mask tokens outside [k0, k1) (and, for PF, past lim)
  if (t0 < k0 || t0 + kChunk > k1 || (PF && t0 + kChunk - 1 > lim_min)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + 16 * (j >> 2) + 4 * kg + (j & 3);
      if (t < k0 || t >= k1 || (PF && t > lim)) sc[j] = -INFINITY;
    }
  }
  float mx = sc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_max = fmaxf(m_run, mx);
  // a column with every token masked so far: subtract 0, so that its weights
  // and alpha come out 0 (not NaN) and its state stays empty
  const float m_new = (PF && m_max == -INFINITY) ? 0.f : m_max;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  bf16x8 pop;
  float psum = 0.f;
  if constexpr (!PAGE) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 p = (__bf16)__builtin_amdgcn_exp2f(sc[j] - m_new);
      pop[j] = p;
      psum += (float)p;   // normalise with the same rounded weights PV uses
    }
  } else {
    const float rvs[2] = {__builtin_amdgcn_rcpf(ch.vs[0]), __builtin_amdgcn_rcpf(ch.vs[1])};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 p = (__bf16)(__builtin_amdgcn_exp2f(sc[j] - m_new) * ch.vs[j >> 2]);
      pop[j] = p;
      psum += (float)p * rvs[j >> 2];
    }
  }
  l_run = l_run * alpha + psum;
  m_run = m_max;
  if (__ballot(alpha != 1.0f) != 0) {
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kg + r);
#pragma unroll
    for (int nb = 0; nb < G::DPL; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nb][r] *= ar[r];
  }
  // V rows as bf16 pairs: rows[j][a] holds head dims DPL*i + 2a, +1 of token j.
  uint32_t rows[8][G::DPL / 2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (!FP8) {
#pragma unroll
      for (int a2 = 0; a2 < G::DPL / 2; ++a2) rows[j][a2] = ch.v[j][a2];
    } else {
#pragma unroll
      for (int u = 0; u < G::VW; ++u) fp8x4_to_bf16x4(ch.v[j][u], rows[j][2 * u], rows[j][2 * u + 1]);
    }
  }
#pragma unroll
  for (int nb = 0; nb < G::DPL; ++nb) {
    const int a2 = nb >> 1;
    u32x4 bv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = rows[2 * q][a2], hi = rows[2 * q + 1][a2];
      bv[q] = (nb & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop, __builtin_bit_cast(bf16x8, bv), acc[nb], 0, 0, 0);
  }
}

// LDS of one tile workgroup.
template <int D>
struct TileSmem {
  float acc[kWaves][kMaxGroup][D];
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
};

// One wave's PV accumulators into LDS: lane (i, kg) holds column 4*kg + r
// (a q head; for multi-token rows a (row, q head) pair) in acc[nb][r], for
// head dim DPL*i + nb (BLOCKED false) or 16*nb + i (true).
template <int D, bool BLOCKED = false>
__device__ inline void store_wave_acc(TileSmem<D>& sm, int wave, int i, int kg, int ncols,
                                      const f32x4 (&acc)[D / 16]) {
  constexpr int DPL = D / 16;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * kg + r;
    if (hh < ncols) {
      if constexpr (BLOCKED) {
#pragma unroll
        for (int nb = 0; nb < DPL; ++nb) sm.acc[wave][hh][16 * nb + i] = acc[nb][r];
      } else {
#pragma unroll
        for (int v4 = 0; v4 < DPL / 4; ++v4) {
          f32x4 o = {acc[4 * v4][r], acc[4 * v4 + 1][r], acc[4 * v4 + 2][r], acc[4 * v4 + 3][r]};
          *reinterpret_cast<f32x4*>(&sm.acc[wave][hh][DPL * i + 4 * v4]) = o;
        }
      }
    }
  }
}

// Cross-wave combine of one item from LDS (per column: running max m,
// weight sum l in units of 2^lse_shift, unnormalised output), then the
// output row (slot -1) or the partial and its natural-log log-sum-exp.
// Column c is packed row qrow0 + c / g, q head h*g + c % g (decode: one row,
// qrow0 = the request).  A column with no unmasked token in this item (only
// possible for multi-token rows) gives o = 0 and lse = -inf, which the merge
// weighs by zero.
template <int D>
__device__ inline void finish_item(const Args& a, const TileSmem<D>& sm, int qrow0, int ncols,
                                   int h, int slot, float vsc, float lse_shift, int tid) {
  const int g = a.group;
  for (int idx = tid; idx < ncols * D; idx += 64 * kWaves) {
    const int hh = idx / D, d = idx - hh * D;
    float M = sm.m[0][hh];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][hh]);
    float lsum = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float wt = __builtin_amdgcn_exp2f(sm.m[ww][hh] - M);
        lsum += wt * sm.l[ww][hh];
        o += wt * sm.acc[ww][hh][d];
      }
    }
    o = lsum > 0.f ? o / lsum * vsc : 0.f;
    const int qr = hh / g;
    const int64_t hq = (int64_t)h * g + (hh - qr * g);
    if (slot < 0) {
      a.out[((int64_t)(qrow0 + qr) * a.n_q_heads + hq) * D + d] = o;
    } else {
      const int64_t prow = ((int64_t)slot * a.qb + qr) * a.n_q_heads + hq;
      a.part_o[prow * D + d] = o;
      if (d == 0)
        a.part_lse[prow] = lsum > 0.f ? (M + log2f(lsum) - lse_shift) * 0.69314718055994531f
                                      : -INFINITY;
    }
  }
}

// New-token prologue, one workgroup (4 waves) per (request b, kv head h):
// q' = RoPE(RMSNorm(q)) for the group's q heads into the workspace (bf16,
// the precision the QK product takes), k' = RoPE(RMSNorm(k_new)) and v_new,
// divided by their scales, stored into cache row len-1.  RMSNorm per head
// over D, then rotate-half RoPE at pos = len-1.  All loads are issued before
// any arithmetic.  Runs before the tile kernel, whose launch then sees the
// written rows.
template <int D, bool FP8>
__global__ __launch_bounds__(256) void hda_prologue_kernel(Args a,
                                                           const int32_t* __restrict__ block_table,
                                                           const int32_t* __restrict__ seq_lens,
                                                           uint16_t* __restrict__ q_out) {
  using G = Geo<D, FP8>;
  constexpr int kHeadsPerWave = kMaxGroup / 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / a.n_kv_heads, h = blockIdx.x % a.n_kv_heads;
  const int g = a.group;
  const int L = seq_lens[b];
  if (L < 1) return;
  const bool act = lane < D / 2;
  const int64_t q0 = ((int64_t)b * a.n_q_heads + (int64_t)h * g) * D;
  const int64_t src = ((int64_t)b * a.n_kv_heads + h) * D;
  // wave w normalises and rotates q heads w, w+4, ...; wave 0 also k and v
  float qx[kHeadsPerWave][2];
#pragma unroll
  for (int j = 0; j < kHeadsPerWave; ++j) {
    const int hh = wave + 4 * j;
    qx[j][0] = act && hh < g ? bf16_bits_to_float(a.q[q0 + (int64_t)hh * D + lane]) : 0.f;
    qx[j][1] = act && hh < g ? bf16_bits_to_float(a.q[q0 + (int64_t)hh * D + lane + D / 2]) : 0.f;
  }
  const bool kv_wave = wave == 0;
  float k0v = act && kv_wave ? bf16_bits_to_float(a.k_new[src + lane]) : 0.f;
  float k1v = act && kv_wave ? bf16_bits_to_float(a.k_new[src + lane + D / 2]) : 0.f;
  const float v0 = act && kv_wave ? bf16_bits_to_float(a.v_new[src + lane]) : 0.f;
  const float v1 = act && kv_wave ? bf16_bits_to_float(a.v_new[src + lane + D / 2]) : 0.f;
  const int pos = L - 1;
  float c = 1.f, s = 0.f;
  if (act) rope_cos_sin(pos, rope_inv_freq(lane, D, a.rope_theta), c, s);
#pragma unroll
  for (int j = 0; j < kHeadsPerWave; ++j) {
    const int hh = wave + 4 * j;
    if (hh < g) {
      norm_rope(qx[j][0], qx[j][1], act, a.q_norm_w, lane, D, a.rms_eps, c, s);
      if (act) {
        q_out[q0 + (int64_t)hh * D + lane] = __builtin_bit_cast(uint16_t, (__bf16)qx[j][0]);
        q_out[q0 + (int64_t)hh * D + lane + D / 2] = __builtin_bit_cast(uint16_t, (__bf16)qx[j][1]);
      }
    }
  }
  if (!kv_wave) return;
  norm_rope(k0v, k1v, act, a.k_norm_w, lane, D, a.rms_eps, c, s);
  const int pidx = pos >> a.log2_ps;
  if (pidx >= a.max_pages) return;
  const int page = block_table[(int64_t)b * a.max_pages + pidx];
  if (page < 0 || page >= a.num_pages || !act) return;
  const int64_t row = (int64_t)page * a.page_stride + (int64_t)h * a.head_stride +
                      (int64_t)(pos & (a.page_size - 1)) * G::RB;
  // the slot is written with the scale it is read with
  float ksc = a.k_scale, vsc = a.v_scale;
  if (a.scale_mode != HDA_SCALE_TENSOR) {
    const int64_t si = a.scale_mode == HDA_SCALE_PAGE ? (int64_t)page * a.n_kv_heads + h : h;
    ksc *= a.k_scales[si];
    vsc *= a.v_scales[si];
  }
  if constexpr (FP8) {
    a.k_pages[row + lane] = (uint8_t)fp8_encode(k0v / ksc);
    a.k_pages[row + lane + D / 2] = (uint8_t)fp8_encode(k1v / ksc);
    if (a.v_dim_major) {   // column pos % ps of the (page, head) slab [D][ps]
      const int64_t col = (int64_t)page * a.page_stride + (int64_t)h * a.head_stride +
                          (pos & (a.page_size - 1));
      a.v_pages[col + (int64_t)lane * a.page_size] = (uint8_t)fp8_encode(v0 / vsc);
      a.v_pages[col + (int64_t)(lane + D / 2) * a.page_size] = (uint8_t)fp8_encode(v1 / vsc);
    } else {
      a.v_pages[row + lane] = (uint8_t)fp8_encode(v0 / vsc);
      a.v_pages[row + lane + D / 2] = (uint8_t)fp8_encode(v1 / vsc);
    }
  } else {
    uint16_t* kp = reinterpret_cast<uint16_t*>(a.k_pages + row);
    uint16_t* vp = reinterpret_cast<uint16_t*>(a.v_pages + row);
    kp[lane] = __builtin_bit_cast(uint16_t, (__bf16)(k0v / ksc));
    kp[lane + D / 2] = __builtin_bit_cast(uint16_t, (__bf16)(k1v / ksc));
    vp[lane] = __builtin_bit_cast(uint16_t, (__bf16)(v0 / vsc));
    vp[lane + D / 2] = __builtin_bit_cast(uint16_t, (__bf16)(v1 / vsc));
  }
}

// One plan item (b, [k0, k1), slot) for kv head h: the waves stream the
// item's chunks, combine in LDS, and write the output (slot -1) or a partial.
//
// Multi-token rows (PF): the item covers nq query rows of request b starting
// at packed row qrow0 and position pos0; column i is row i / g, q head
// h*g + i % g, with causal limit pos0 + i / g.  Decode is nq = 1, qrow0 = b.
// A plan item's range against its request's length L on the device: cut at
// L (a plan built for longer lengths then leaves the tokens past L out; an
// item wholly past L becomes empty) and return the check bits --
// HDA_CHECK_PAST_LEN when the item reached past L, HDA_CHECK_SHORT when the
// request's last item ends before L (the plan was built for shorter
// lengths; those tokens stay unattended).
__device__ inline int cut_at_len(int& k1, int L, bool last) {
  if (k1 > L) {
    k1 = L;
    return HDA_CHECK_PAST_LEN;
  }
  return last && k1 < L ? HDA_CHECK_SHORT : 0;
}

// The workgroup's check word (one writer per word; every launch rewrites it).
__device__ inline void write_check(const Args& a, int bits, int tid) {
  if (a.check && tid == 0) a.check[blockIdx.x] = bits;
}

// Coverage counting (debug launches only): each token of chunk c inside the
// item's range [k0, k1) -- the tokens the chunk's softmax keeps -- adds one
// visit to its cache row (physical page, row in page) for kv head h.
template <int CH>
__device__ inline void count_visits(const Args& a, const int32_t* __restrict__ block_table, int b,
                                    int h, int c, int k0, int k1, int lane) {
  if (lane >= CH) return;
  const int t = c * CH + lane;
  if (t < k0 || t >= k1) return;
  const int pidx = t >> a.log2_ps;
  const int page = pidx < a.max_pages ? block_table[(int64_t)b * a.max_pages + pidx] : -1;
  if (page < 0 || page >= a.num_pages) return;
  atomicAdd(&a.cover[((int64_t)page * a.page_size + (t & (a.page_size - 1))) * a.n_kv_heads + h],
            1);
}

template <int D, bool FP8, bool PAGE, bool PF, bool COVER = false>
__device__ inline void process_item(const Args& a, const int32_t* __restrict__ block_table,
                                    TileSmem<D>& sm, int b, int k0, int k1, int slot, int L,
                                    int qrow0, int nq, int pos0, int h, int wave, int lane,
                                    int tid) {
  using G = Geo<D, FP8>;
  const int i = lane & 15, kg = lane >> 4;
  const int g = a.group;
  // score and output scales of this kv head (per-page factors are applied
  // per half-chunk instead)
  float qk = a.qk_scale_log2, vsc = a.v_scale;
  if (!PAGE && a.scale_mode == HDA_SCALE_HEAD) {
    qk *= a.k_scales[h];
    vsc *= a.v_scales[h];
  }
    const int qr = PF ? i / g : 0;
    const int hh = i - qr * g;
    const bool col_live = PF ? qr < nq : i < g;
    const int lim = col_live ? pos0 + qr : 0x7fffffff;   // causal limit of column i
    const int64_t qbase = ((int64_t)(qrow0 + qr) * a.n_q_heads + (int64_t)h * g + hh) * D;

    // Chunks c_first + wave, + kWaves, ...; two register sets in flight.
    const int c_last = (k1 - 1) / kChunk;
    int c = k0 / kChunk + wave;
    // uniform per wave; an item left empty by the cut at the device length
    // computes nothing and writes an empty partial (o = 0, lse = -inf)
    const bool has_chunks = k0 < k1 && c <= c_last;
    Chunk<D, FP8> ring[G::NBUF];
    __amdgpu_buffer_rsrc_t kr[2], vr[2];

    // q operand (MFMA B): lane (i, kg) holds column i, dims qk_dim(s, kg) + 0..7.
    bf16x8 qop[G::STEPS];
#pragma unroll
    for (int s2 = 0; s2 < G::STEPS; ++s2) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col_live) v = *reinterpret_cast<const u32x4*>(a.q + qbase + qk_dim<FP8>(s2, kg));
      qop[s2] = __builtin_bit_cast(bf16x8, v);
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[G::DPL];
#pragma unroll
    for (int nb = 0; nb < G::DPL; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (has_chunks) {
      // A ring of G::NBUF register sets: the loads of the chunk NBUF-1 steps
      // ahead are issued before this chunk's math (the scheduling barrier
      // keeps the compiler from sinking them below it).
#pragma unroll
      for (int k = 0; k < G::NBUF - 1; ++k) {
        const int ck = c + k * kWaves;
        chunk_rsrc<D, FP8, PAGE>(a, block_table, b, L, h, ck, ck <= c_last, kr, vr, ring[k]);
        issue_chunk<D, FP8>(ring[k], kr, vr, i, kg);
      }
      bool done = false;
      while (!done) {
#pragma unroll
        for (int k = 0; k < G::NBUF; ++k) {
          const int cn = c + (G::NBUF - 1) * kWaves;
          const int nx = (k + G::NBUF - 1) % G::NBUF;
          chunk_rsrc<D, FP8, PAGE>(a, block_table, b, L, h, cn, cn <= c_last, kr, vr, ring[nx]);
          issue_chunk<D, FP8>(ring[nx], kr, vr, i, kg);
          __builtin_amdgcn_sched_barrier(0);
          compute_chunk<D, FP8, PAGE, PF>(ring[k], qop, c, k0, k1, lim, pos0, qk, kg, m_run,
                                          l_run, acc);
          if constexpr (COVER) count_visits<kChunk>(a, block_table, b, h, c, k0, k1, lane);
          c += kWaves;
          if (c > c_last) {
            done = true;
            break;
          }
        }
      }
    }


    // Combine the waves of this workgroup.
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    // the previous item's combine has finished reading this LDS
    __syncthreads();
    if (kg == 0) {
      sm.m[wave][i] = m_run;
      sm.l[wave][i] = l_tot;
    }
    const int ncols = PF ? nq * g : g;
    store_wave_acc<D>(sm, wave, i, kg, ncols, acc);
    __syncthreads();
    finish_item<D>(a, sm, qrow0, ncols, h, slot, vsc, 0.f, tid);
}

// ---- native-fp8 products: fp8 cache, dim-major V pages, D = 128 ----
//
// QK^T and PV take the fp8 codes as MFMA operands directly.  A wave takes
// 64-token chunks (one page of 64, or a 64-token run of a larger page).
//   QK: four 16-token M blocks, each two v_mfma_scale_f32_16x16x128_f8f6f4
//       of K rows against q quantised per q head (s_q = amax / 448) as an
//       E4M3 high part (operand scale 2^0) plus an E4M3 residual x 16
//       (operand scale 2^-4).  Row m of block mb is token
//       16*(m/4) + 4*mb + m%4, so lane (i, kg) ends up with the scores of
//       q head i for its 16 consecutive tokens 16*kg .. 16*kg+15.
//   PV: the softmax weights, shifted by 2^8 and kept as an E4M3 value plus
//       an E4M3 residual (two products into one accumulator), against V
//       codes read from dim-major pages, where those 16 tokens of one head
//       dim are 16 consecutive bytes: two v_mfma_f32_16x16x32_fp8_fp8 per
//       16-dim block and part (lane i takes dim 16*nb + i), no transposes.
//       The weight sum comes from the same rounded weights through more
//       MFMAs against a block of 1.0 codes.
constexpr int kChunkN = 64;
constexpr uint64_t kFp8Ones = 0x3838383838383838ull;   // eight E4M3 1.0 codes

typedef __attribute__((ext_vector_type(8))) int i32x8;

struct ChunkN {
  u32x4 k[4][2];   // K: 32 dims of one token row per lane, per 16-token block
  u32x4 v[8];      // V: 16 tokens of head dim 16*nb + i per lane, nb = 0..7
};

// Buffer resources of chunk c of (request b, kv head h): the 64 K rows from
// token t, and the V slab from token column t%ps of every head-dim row.
// Returns the number of rows below len (0 for a chunk without a page).
__device__ inline int chunk_rsrc_n(const Args& a, const int32_t* __restrict__ block_table, int b,
                                   int L, int h, int c, bool live, __amdgpu_buffer_rsrc_t& kr,
                                   __amdgpu_buffer_rsrc_t& vr) {
  const int t = c * kChunkN;
  int rows = L - t;
  rows = rows > kChunkN ? kChunkN : rows;
  int64_t koff = 0, voff = 0;
  int kbytes = 0, vbytes = 0;
  if (live && rows > 0) {
    const int pidx = t >> a.log2_ps;
    if (pidx < a.max_pages) {
      const int page = block_table[(int64_t)b * a.max_pages + pidx];
      if (page >= 0 && page < a.num_pages) {
        const int64_t slab = (int64_t)page * a.page_stride + (int64_t)h * a.head_stride;
        const int tin = t & (a.page_size - 1);
        koff = slab + (int64_t)tin * 128;
        kbytes = kChunkN * 128;
        voff = slab + tin;
        vbytes = 127 * a.page_size + kChunkN;   // dims 0..127, 64 columns from tin
      }
    }
  }
  kr = make_rsrc(a.k_pages + koff, kbytes);
  vr = make_rsrc(a.v_pages + voff, vbytes);
  return kbytes > 0 ? rows : 0;
}

// One lane offset per tensor serves every load of a chunk; the per-block
// parts are wave-uniform and go in the scalar offset, which the buffer range
// check leaves out.  Both stay inside the (page, kv head) slab by
// construction (a 64-token chunk lies within one page of >= 64 tokens).  K
// rows past len may thus be read: they only feed the scores of tokens past
// len, which are overwritten with -inf.  V columns past len are masked after
// the load.  A chunk without a page reads zeros (empty resource).
__device__ inline void issue_chunk_n(ChunkN& ch, const __amdgpu_buffer_rsrc_t& kr,
                                     const __amdgpu_buffer_rsrc_t& vr, int koff, int voff,
                                     int ps) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      ch.k[mb][u] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, koff, 4 * 128 * mb + 64 * u, kStreamAux));
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    ch.v[nb] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, voff, 16 * nb * ps, kStreamAux));
}

__device__ inline uint64_t pack64(uint32_t lo, uint32_t hi) {
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

// One 64-token chunk: scores, online-softmax update, acc += P8 V8, and the
// rounded weights' sum into lacc (both in units of 2^8).  qs = score scale of
// lane i's q head in log2 units (sm_scale * k scale * s_q * log2 e).
__device__ inline void compute_chunk_n(const ChunkN& ch, const i32x8& qop, const i32x8& qlo,
                                       int c, int k0, int k1,
                                       int rows, float qs, int kg, float& m_run, f32x4 (&acc)[8],
                                       f32x4& lacc) {
  float sc[16];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const i32x8 kop = {(int)ch.k[mb][0][0], (int)ch.k[mb][0][1], (int)ch.k[mb][0][2],
                       (int)ch.k[mb][0][3], (int)ch.k[mb][1][0], (int)ch.k[mb][1][1],
                       (int)ch.k[mb][1][2], (int)ch.k[mb][1][3]};
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    // K q_hi, then + K q_lo with q_lo's operand scale 2^-4 (E8M0 code 123)
    f32x4 sacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qop, z, 0, 0, 0, 127, 0,
                                                                 127);
    sacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qlo, sacc, 0, 0, 0, 127, 0, 123);
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[4 * mb + r] = sacc[r] * qs;
  }
  const int t0 = c * kChunkN;
  if (t0 < k0 || t0 + kChunkN > k1) {   // partial chunk: mask tokens outside [k0, k1)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int t = t0 + 16 * kg + x;
      if (t < k0 || t >= k1) sc[x] = -INFINITY;
    }
  }
  float mx = sc[0];
#pragma unroll
  for (int x = 1; x < 16; ++x) mx = fmaxf(mx, sc[x]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  // weights z = p 2^8 as a = E4M3(z) plus b = E4M3(z - a) (the difference
  // is exact in float32): both go through PV into the same accumulator, so
  // the product sees a + b, within 2^-8 z + 2^-10 of z where a alone is
  // within 2^-4 z
  uint32_t pw[4], pr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = __builtin_amdgcn_exp2f(sc[4 * q + j] - m_new) * 256.f;
    const int x = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
    const int a = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], x, true);
    pw[q] = (uint32_t)a;
    const float r0 = e[0] - __builtin_amdgcn_cvt_f32_fp8(a, 0);
    const float r1 = e[1] - __builtin_amdgcn_cvt_f32_fp8(a, 1);
    const float r2 = e[2] - __builtin_amdgcn_cvt_f32_fp8(a, 2);
    const float r3 = e[3] - __builtin_amdgcn_cvt_f32_fp8(a, 3);
    const int y = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
    pr[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, y, true);
  }
  m_run = m_new;
  if (__ballot(alpha != 1.0f) != 0) {
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kg + r);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nb][r] *= ar[r];
#pragma unroll
    for (int r = 0; r < 4; ++r) lacc[r] *= ar[r];
  }
  // weights of tokens 16*kg + 8*ks + j, j = 0..7, for K steps ks = 0, 1
  // (p: the E4M3 weights, r: their residuals)
  const long p0 = (long)pack64(pw[0], pw[1]);
  const long p1 = (long)pack64(pw[2], pw[3]);
  const long r0 = (long)pack64(pr[0], pr[1]);
  const long r1 = (long)pack64(pr[2], pr[3]);
  // V columns past len hold anything (a NaN code times a zero weight would
  // still poison the sum): zero them in the last chunk of a request
  uint32_t vm[4] = {~0u, ~0u, ~0u, ~0u};
  if (rows < kChunkN) {
    int nv = rows - 16 * kg;
    nv = nv < 0 ? 0 : (nv > 16 ? 16 : nv);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int bq = nv - 4 * q;
      vm[q] = bq >= 4 ? ~0u : (bq <= 0 ? 0u : ((1u << (8 * bq)) - 1u));
    }
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const u32x4 v = ch.v[nb];
    const long v0 = (long)pack64(v[0] & vm[0], v[1] & vm[1]);
    const long v1 = (long)pack64(v[2] & vm[2], v[3] & vm[3]);
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(p0, v0, acc[nb], 0, 0, 0);
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(p1, v1, acc[nb], 0, 0, 0);
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(r0, v0, acc[nb], 0, 0, 0);
    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(r1, v1, acc[nb], 0, 0, 0);
  }
  lacc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(p0, (long)kFp8Ones, lacc, 0, 0, 0);
  lacc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(p1, (long)kFp8Ones, lacc, 0, 0, 0);
  lacc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(r0, (long)kFp8Ones, lacc, 0, 0, 0);
  lacc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(r1, (long)kFp8Ones, lacc, 0, 0, 0);
}

// One plan item in the native-fp8 mode (see process_item for the shape of
// the loop and the combine).
template <bool COVER = false>
__device__ inline void process_item_fp8n(const Args& a, const int32_t* __restrict__ block_table,
                                         TileSmem<128>& sm, int b, int k0, int k1, int slot,
                                         int L, int h, int wave, int lane, int tid) {
  const int i = lane & 15, kg = lane >> 4;
  const int g = a.group;
  float qk = a.qk_scale_log2, vsc = a.v_scale;
  if (a.scale_mode == HDA_SCALE_HEAD) {
    qk *= a.k_scales[h];
    vsc *= a.v_scales[h];
  }
  // q head i in E4M3: lane (i, kg) holds dims 16*kg + 0..15 and 64 + 16*kg +
  // 0..15, the order of the K rows' operand; s_q = amax / 448 (1 for a zero
  // row), codes round-to-nearest-even from q / s_q in float32
  const int64_t qrow = ((int64_t)b * a.n_q_heads + (int64_t)h * g + i) * 128;
  float qv[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (i < g)
      raw = *reinterpret_cast<const u32x4*>(a.q + qrow + 64 * (u >> 1) + 16 * kg + 8 * (u & 1));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[8 * u + 2 * e] = __uint_as_float(raw[e] << 16);
      qv[8 * u + 2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int x = 0; x < 32; ++x) amax = fmaxf(amax, fabsf(qv[x]));
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const float s_q = amax > 0.f ? amax / 448.0f : 1.0f;
  // q / s_q as a high part and a residual: hi = E4M3(x), lo = E4M3(16 (x -
  // hi)) (the difference is exact in float32), so the score uses
  // s_q (hi + lo / 16) -- relative error about 2^-8 instead of E4M3's 2^-4,
  // the quantisation that dominated this mode's error.  The split is the
  // Router GEMM's (a high part plus a residual kept at a larger scale and
  // scaled back in the product) applied to q; the two products share the K
  // operand, the second taking the 2^-4 as its operand scale.
  i32x8 qop, qlo;
#pragma unroll
  for (int dw = 0; dw < 8; ++dw) {
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = fminf(fmaxf(qv[4 * dw + e] / s_q, -448.f), 448.f);
    const int h01 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    const int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], h01, true);
    qop[dw] = hi;
    const float r0 = (x[0] - __builtin_amdgcn_cvt_f32_fp8(hi, 0)) * 16.f;
    const float r1 = (x[1] - __builtin_amdgcn_cvt_f32_fp8(hi, 1)) * 16.f;
    const float r2 = (x[2] - __builtin_amdgcn_cvt_f32_fp8(hi, 2)) * 16.f;
    const float r3 = (x[3] - __builtin_amdgcn_cvt_f32_fp8(hi, 3)) * 16.f;
    const int l01 = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
    qlo[dw] = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, l01, true);
  }
  const float qs = qk * s_q;

  const int c_last = (k1 - 1) / kChunkN;
  int c = k0 / kChunkN + wave;
  const bool has_chunks = k0 < k1 && c <= c_last;
  ChunkN ring[2];
  int rows_of[2];
  __amdgpu_buffer_rsrc_t kr, vr;
  // lane (i, kg): K row 16*(i/4) + i%4 of M block 0 (block mb adds 4*mb
  // rows), bytes 16*kg of each 64-byte half; V row (head dim) i of each
  // 16-dim block (block nb adds 16*nb rows: one load covers 16 whole rows),
  // tokens 16*kg
  const int koff = (16 * (i >> 2) + (i & 3)) * 128 + 16 * kg;
  const int voff = i * a.page_size + 16 * kg;
  float m_run = -INFINITY;
  f32x4 acc[8], lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (has_chunks) {
    rows_of[0] = chunk_rsrc_n(a, block_table, b, L, h, c, true, kr, vr);
    issue_chunk_n(ring[0], kr, vr, koff, voff, a.page_size);
    bool done = false;
    while (!done) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int cn = c + kWaves;
        rows_of[1 - k] = chunk_rsrc_n(a, block_table, b, L, h, cn, cn <= c_last, kr, vr);
        issue_chunk_n(ring[1 - k], kr, vr, koff, voff, a.page_size);
        __builtin_amdgcn_sched_barrier(0);
        compute_chunk_n(ring[k], qop, qlo, c, k0, k1, rows_of[k], qs, kg, m_run, acc, lacc);
        if constexpr (COVER) count_visits<kChunkN>(a, block_table, b, h, c, k0, k1, lane);
        c += kWaves;
        if (c > c_last) {
          done = true;
          break;
        }
      }
    }
  }

  // the previous item's combine has finished reading this LDS
  __syncthreads();
  if (kg == 0) sm.m[wave][i] = m_run;
  if (i == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * kg + r < g) sm.l[wave][4 * kg + r] = lacc[r];
  }
  store_wave_acc<128, true>(sm, wave, i, kg, g, acc);
  __syncthreads();
  finish_item<128>(a, sm, b, g, h, slot, vsc, 8.f, tid);
}

// ---- multi-token rows with the K/V chunk shared through LDS ----
//
// For blocks of more than 16/g query rows: the workgroup (NW waves) loads
// each K/V stage (SUB chunks of 32 tokens) of the item once into LDS and
// all waves multiply it.  The block's rows come in tiles of unit = 16/g
// rows (16 columns, the decode kernel's column shape); wave w owns tiles
// w, w + NW, ... (TPW of them).  The bytes requested from memory per item
// drop by the number of busy tiles; each wave reads a chunk's operands from
// LDS once for all its tiles.  Two stages alternate: the next one is loaded
// into registers while the current one is multiplied (across items too: an
// item's last stage overlaps the loads of the next item's first).
//
// LDS holds each chunk in bf16 (fp8 pages are decoded once, when stored),
// laid out so that every MFMA operand is one 16-byte read per lane and no
// read has a bank conflict.  (gfx950 serves a 16-byte read 16 lanes at a
// time, and measured conflict-free only when lanes 0-7 and lanes 8-15 of
// each group each cover one aligned half of the 64 banks: rows padded by 16
// bytes, which spread a group over all banks but straddle the halves, took
// twice the cycles.)
//   k   K rows [token][D]; 16-byte quad q of token row r sits at
//       k_off(r, q): for D = 128, rows of 256 bytes with the quad XOR-ed
//       by r mod 16; for D = 64, rows r and r + 8 of each 16 share 256-byte
//       lines, quad q of row r in half (q / 4) ^ (r / 8 mod 2) at position
//       (r ^ q) mod 8.  Lane (i, kg) of QK step s reads quad 4s + kg of
//       token row 16*hf + i.
//   vt  V transposed, dim-major: head dim d on row rho = 16 * (d % DPL) +
//       d / DPL and token t at position 8 * ((t % 16) / 4) + 4 * (t / 16) +
//       t % 4 -- the order of the PV weights' k index -- stored by blocks of
//       16 rows, each block as 4 runs (one per 8 positions) of its 16 rows'
//       16-byte pieces: lane (i, kg) of PV block nb reads the contiguous
//       piece 16 * i of run kg of block nb.
// The transpose happens when a stage is stored: each storing thread holds
// the same 16-byte column of two adjacent tokens, and writes dword pairs
// (token t, t+1) of each dim.
//
// PV is computed transposed, O^T += V^T P^T (V^T from LDS as MFMA A, the
// weights as B), which leaves column i of the output in lane (i, kg), the
// lane that holds column i's scores: the online-softmax rescale is
// lane-local.
template <int D, int SUB>
struct alignas(16) SharedStage {
  static_assert(D == 64 || D == 128, "stage layouts for head dims 64 and 128");
  uint8_t k[SUB * kChunk * 2 * D];              // SUB chunks of K rows
  uint8_t vt[SUB][D * 2 * kChunk];              // V^T of each chunk
  // byte offset of 16-byte quad q of token row r
  __device__ static int k_off(int r, int q) {
    if constexpr (D == 128) {
      return r * 256 + 16 * (q ^ (r & 15));
    } else {
      return (r >> 4) * 2048 + (r & 7) * 256 +
             16 * (8 * ((q >> 2) ^ ((r >> 3) & 1)) + ((r ^ q) & 7));
    }
  }
  // byte offset of (V^T row rho, token position pos) within a chunk
  __device__ static int vt_off(int rho, int pos) {
    return 1024 * (rho >> 4) + 256 * (pos >> 3) + 16 * (rho & 15) + 2 * (pos & 7);
  }
};

// 32-token chunks per LDS stage of the shared kernel (one stage in flight
// while the other is multiplied; four chunks per stage measured slower
// than two).
constexpr int kSharedSub = 2;

// Weights of the shared kernel's lazily rescaled softmax stay below 2^8.
constexpr float kLazyLog2 = 8.f;

// Position of token t (0..31) of a chunk in a V^T row.
__device__ inline int vt_pos(int t) {
  return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3);
}

// S^T = K Q^T for one chunk and one tile from LDS operands kf (K, MFMA A,
// per 16-token half and QK step) -- qk_scores -- then the online-softmax
// update, which yields the tile's PV weights (MFMA B layout of P^T; lane
// (i, kg) holds column i).  The PV accumulators hold column i in lane (i, kg),
// so alpha is lane-local.  With per-page factors the update is
// softmax_update's, and l_run holds this lane's share of the column sum.
template <int D>
__device__ inline void qk_scores(const bf16x8 (&kf)[2][D / 32], const bf16x8 (&qop)[D / 32],
                                 f32x4 (&sacc)[2]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    sacc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      sacc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[hf][s], qop[s], sacc[hf], 0, 0, 0);
  }
}

// The update without per-page factors, for all TPW tiles of a wave at once
// (one branch per mask and one for the rescale serve every tile, so that the
// tiles' dependency chains interleave; tiles that see none of the chunk come
// out with weights 0 and unchanged state).  The score scale is one number:
// the max is taken over the raw products (the scale is positive) and each
// weight is exp2(s * scale - m) with one fused multiply-add, m being a
// lazily raised reference (any reference gives the same quotient acc / l, up
// to rounding): it moves only when a column's maximum passes it by more than
// kLazyLog2, so the weights stay below 2^kLazyLog2 and most chunks skip the
// rescale.  It starts at -FLT_MAX: the first visible token moves it, and a
// column with every token masked so far gets weights 0, not NaN.  The
// column's weight sum is one more MFMA, a block of 1.0 times the rounded
// weights (the exact fp32 sum of what PV multiplies) accumulated in l_acc,
// whose element 0 holds the whole column's sum.  Masks come in two uniform
// branches, taken only by the chunks that need them: tokens before k0 (an
// item starting inside the chunk), and tokens past a column's last visible
// one, hi = min(k1 - 1, causal limit); each element's offset 16 (j / 4) +
// j % 4 is a constant compared with a per-lane threshold (the threshold of
// the first through readfirstlane, a convergent operation, which keeps the
// tests inside the branch).
template <int D, int TPW>
__device__ inline void softmax_tiles(f32x4 (&sacc)[TPW][2], int c, int k0, int k1,
                                     const int (&lim)[TPW], const int (&lim_min)[TPW],
                                     float qk_scale_log2, int kg, float (&m_run)[TPW],
                                     f32x4 (&l_acc)[TPW], f32x4 (&acc)[TPW][D / 16],
                                     bf16x8 (&pop)[TPW]) {
  constexpr int DPL = D / 16;
  float sc[TPW][8];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) sc[t][j] = sacc[t][j >> 2][j & 3];
  const int t0 = c * kChunk;
  if (t0 < k0) {
    const int d = __builtin_amdgcn_readfirstlane(k0 - t0) - 4 * kg;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (16 * (j >> 2) + (j & 3) < d) sc[t][j] = -INFINITY;
  }
  int hi_min = k1 - 1;
#pragma unroll
  for (int t = 0; t < TPW; ++t) hi_min = min(hi_min, lim_min[t]);
  if (t0 + kChunk - 1 > hi_min) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int r = min(k1 - 1, lim[t]) - t0 - 4 * kg;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (16 * (j >> 2) + (j & 3) > r) sc[t][j] = -INFINITY;
    }
  }
  const float inf = opaque_inf();
  float mx[TPW];
  bool grow = false;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    mx[t] = qmax(qmax(qmax(sc[t][0], sc[t][1], inf), qmax(sc[t][2], sc[t][3], inf), inf),
                 qmax(qmax(sc[t][4], sc[t][5], inf), qmax(sc[t][6], sc[t][7], inf), inf), inf);
    mx[t] = kg_reduce_qmax(mx[t], inf) * qk_scale_log2;
    grow = grow || mx[t] > m_run[t] + kLazyLog2;
  }
  // the reference moves for every tile when any column needs it
  if (__ballot(grow) != 0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const float m_new = fmaxf(m_run[t], mx[t]);
      const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_new);
      l_acc[t][0] *= alpha;
      m_run[t] = m_new;
#pragma unroll
      for (int nb = 0; nb < DPL; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][nb][r] *= alpha;
    }
  }
  const bf16x8 ones = __builtin_bit_cast(
      bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pop[t][j] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][j], qk_scale_log2, -m_run[t]));
    l_acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop[t], l_acc[t], 0, 0, 0);
  }
}

// Sixteen-bit halves: (lo of a, lo of b) and (hi of a, hi of b).
__device__ inline uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ inline uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Register-staged loads of one LDS stage (SUB chunks of K and V) of the
// shared kernel, by all NW waves.  Loads come in pairs: V pair v = (column
// v % PPR of tokens 2 (v / PPR) and +1), then K pair k (two 16-byte pieces,
// task_piece); task tau = tid + NT u.  The counts are multiples of 64, so a wave's tasks are all of
// one kind.  Branch-free: a load whose token is past len or has no page
// reads a valid address (page 0) and is zeroed when stored (ok bit 2u + m),
// so the wait before a store counts only that stage's loads.
template <int D, bool FP8, bool PAGE, int NW, int SUB>
struct StageLoader {
  using G = Geo<D, FP8>;
  static constexpr int DPL = D / 16;
  static constexpr int NT = 64 * NW;
  static constexpr int STOK = SUB * kChunk;          // tokens per stage
  static constexpr int PPR = G::RB / 16;             // 16-byte pieces per cached token row
  static constexpr int VPAIRS = STOK / 2 * PPR;
  static constexpr int TASKS = VPAIRS + STOK * PPR / 2;
  static constexpr int TPT = (TASKS + NT - 1) / NT;
  static constexpr int HALVES = 2 * SUB;             // 16-token groups of a stage
  static_assert(VPAIRS % 64 == 0 && TASKS % 64 == 0, "wave-uniform task kinds");
  // When the counts divide by the thread count, slot u holds one kind of
  // task for every thread; deciding it at compile time keeps every load
  // outside branches (a conditional load makes the waits before the stores
  // conservative).
  static constexpr bool kStaticKinds = VPAIRS % NT == 0 && TASKS % NT == 0;
  // Both loads of a task slot fall in one 16-token group in every lane of a
  // wave when a cache row has at least 8 pieces: V pairs of a wave then span
  // at most 16 tokens, and a K slot's rows 8 (task_piece).
  static constexpr bool kUniformGroup = PPR >= 8;
  __device__ static bool is_v_task(int u, int tau) {
    return kStaticKinds ? NT * u < VPAIRS : tau < VPAIRS;
  }
  __device__ static bool live_task(int u, int tau) {
    return kStaticKinds ? NT * u < TASKS : tau < TASKS;
  }
  // Piece m of K task k: token row and 16-byte column of the cache row.
  // For bf16 rows of 16 pieces (D = 128) the 16 tasks 16a .. 16a + 15 take
  // rows 2a (m = 0) and 2a + 1 (m = 1), task 16a + x the piece that lands
  // on quad x of the swizzled row, so that each store fills a row's 256
  // bytes; otherwise task k takes pieces 2k and 2k + 1 in row order.
  __device__ static void task_piece(int k, int m, int& row, int& col) {
    if constexpr (!FP8 && PPR == 16) {
      row = 2 * (k >> 4) + m;
      col = (k & 15) ^ (row & 15);
    } else {
      const int p = 2 * k + m;
      row = p / PPR;
      col = p % PPR;
    }
  }
  u32x4 st[TPT][2];
  uint32_t st_ok;
  float sks[HALVES], svs[HALVES];                    // page factors of the groups

  // the stage from chunk c of request b (length L), kv head h
  __device__ inline void fetch(const Args& a, const int32_t* __restrict__ block_table, int b,
                               int L, int h, int c, int tid) {
    const int t0 = c * kChunk;
    // page of 16-token group hf of the stage (page 0 when the group has no
    // valid page: its loads are then zeroed when stored)
    auto group_page = [&](int hf, bool& pok) {
      const int t = t0 + 16 * hf;
      const int pidx = t >> a.log2_ps;
      const int pg = (t < L && pidx < a.max_pages) ? block_table[(int64_t)b * a.max_pages + pidx] : -1;
      pok = pg >= 0 && pg < a.num_pages;
      return pok ? pg : 0;
    };
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf) {
      sks[hf] = svs[hf] = 1.f;
      if constexpr (PAGE) {
        bool pok;
        const int pg = group_page(hf, pok);
        if (pok) {
          sks[hf] = a.k_scales[(int64_t)pg * a.n_kv_heads + h];
          svs[hf] = a.v_scales[(int64_t)pg * a.n_kv_heads + h];
        }
      }
    }
    // rows and columns of every slot's loads
    int row[TPT][2], col[TPT][2];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int tau = tid + NT * u;
      if (is_v_task(u, tau)) {
        row[u][0] = 2 * (tau / PPR);
        row[u][1] = row[u][0] + 1;
        col[u][0] = col[u][1] = tau % PPR;
      } else {
#pragma unroll
        for (int m = 0; m < 2; ++m) task_piece(tau - VPAIRS, m, row[u][m], col[u][m]);
      }
    }
    st_ok = 0u;
    if constexpr (kUniformGroup) {
      // both loads of a slot, in every lane of the wave, fall in one 16-token
      // group: one page lookup per slot (all slots' lookups issued together),
      // a uniform slab address and a 32-bit offset per lane
      int pg[TPT];
      bool pok[TPT];
#pragma unroll
      for (int u = 0; u < TPT; ++u)
        pg[u] = group_page(__builtin_amdgcn_readfirstlane(row[u][0] >> 4), pok[u]);
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int tau = tid + NT * u;
        if (!live_task(u, tau)) break;               // uniform per wave
        const uint8_t* slab = (is_v_task(u, tau) ? a.v_pages : a.k_pages) +
                              (int64_t)pg[u] * a.page_stride + (int64_t)h * a.head_stride;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int t = t0 + row[u][m];
          const uint32_t in_page = (uint32_t)((t & (a.page_size - 1)) * G::RB + 16 * col[u][m]);
          st[u][m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(slab + in_page));
          st_ok |= (t < L && pok[u] ? 1u : 0u) << (2 * u + m);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int tau = tid + NT * u;
        if (!live_task(u, tau)) break;               // uniform per wave
        const uint8_t* pool = is_v_task(u, tau) ? a.v_pages : a.k_pages;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int t = t0 + row[u][m];
          bool pok;
          const int pg = group_page(row[u][m] >> 4, pok);
          const int64_t off = (int64_t)pg * a.page_stride + (int64_t)h * a.head_stride +
                              (int64_t)(t & (a.page_size - 1)) * G::RB + 16 * col[u][m];
          st[u][m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pool + off));
          st_ok |= (t < L && pok ? 1u : 0u) << (2 * u + m);
        }
      }
    }
  }
  // Store the registers as a stage (bf16, transposed V).
  __device__ inline void put(SharedStage<D, SUB>& ss, int tid) const {
    using SS = SharedStage<D, SUB>;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int tau = tid + NT * u;
      if (!live_task(u, tau)) break;
      u32x4 x[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        x[m] = ((st_ok >> (2 * u + m)) & 1u) ? st[u][m] : u32x4{0u, 0u, 0u, 0u};
      if (is_v_task(u, tau)) {
        const int col = tau % PPR;
        // tokens t, t + 1 (one dword) of every V^T row their column covers
        const int t = 2 * (tau / PPR);
        uint8_t* dst = ss.vt[t / kChunk];
        const int pos = vt_pos(t % kChunk);
        if constexpr (!FP8) {
          // dims 8 col + e: dword (token t, token t + 1)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = 8 * col + e;
            const uint32_t w = (e & 1) ? pair_hi(x[0][e >> 1], x[1][e >> 1])
                                       : pair_lo(x[0][e >> 1], x[1][e >> 1]);
            *reinterpret_cast<uint32_t*>(dst + SS::vt_off(16 * (d % DPL) + d / DPL, pos)) = w;
          }
        } else {
          // dims 16 col + e, decoded: bf16 pairs (4k, 4k+1), (4k+2, 4k+3)
#pragma unroll
          for (int kq = 0; kq < 4; ++kq) {
            uint32_t a0, a1, b0, b1;
            fp8x4_to_bf16x4(x[0][kq], a0, a1);
            fp8x4_to_bf16x4(x[1][kq], b0, b1);
            const uint32_t w[4] = {pair_lo(a0, b0), pair_hi(a0, b0), pair_lo(a1, b1),
                                   pair_hi(a1, b1)};
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              const int d = 16 * col + 4 * kq + e2;
              *reinterpret_cast<uint32_t*>(dst + SS::vt_off(16 * (d % DPL) + d / DPL, pos)) = w[e2];
            }
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          int row, col;
          task_piece(tau - VPAIRS, m, row, col);
          if constexpr (!FP8) {
            *reinterpret_cast<u32x4*>(ss.k + SS::k_off(row, col)) = x[m];
          } else {
            uint32_t w[8];
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) fp8x4_to_bf16x4(x[m][kq], w[2 * kq], w[2 * kq + 1]);
            *reinterpret_cast<u32x4*>(ss.k + SS::k_off(row, 2 * col)) = u32x4{w[0], w[1], w[2], w[3]};
            *reinterpret_cast<u32x4*>(ss.k + SS::k_off(row, 2 * col + 1)) = u32x4{w[4], w[5], w[6], w[7]};
          }
        }
      }
    }
  }
};

// Item (b, [k0, k1), slot) of row block (qrow0, nq rows, first position
// pos0) for kv head h.  On entry the loader holds the item's first stage in
// registers; during its last stage it fetches the first stage of the next
// item (next_b, next_L, next_c: request, length, first chunk) when
// has_next, so that stage's loads overlap this item's arithmetic.
template <int D, bool FP8, bool PAGE, int NW, int TPW, int SUB>
__device__ inline void process_item_shared(const Args& a, const int32_t* __restrict__ block_table,
                                           SharedStage<D, SUB> (&buf)[2],
                                           StageLoader<D, FP8, PAGE, NW, SUB>& ld, int b, int k0,
                                           int k1, int slot, int L, int qrow0, int nq, int pos0,
                                           int h, bool has_next, int next_b, int next_L,
                                           int next_c, int wave, int lane, int tid) {
  using SS = SharedStage<D, SUB>;
  constexpr int DPL = D / 16, STEPS = D / 32;
  constexpr int HALVES = 2 * SUB;
  // sixteen waves of one tile: K and V fragments read half at a time
  constexpr bool kHalves = NW == 16 && !PAGE;
  const int i = lane & 15, kg = lane >> 4;
  const int g = a.group;
  const int unit = kMaxGroup / g;                    // rows per tile
  float qk = a.qk_scale_log2, vsc = a.v_scale;
  if (!PAGE && a.scale_mode == HDA_SCALE_HEAD) {
    qk *= a.k_scales[h];
    vsc *= a.v_scales[h];
  }
  const int qr = i / g, hh = i - qr * g;
  int r0[TPW], nqw[TPW], lim[TPW], lim_min[TPW], lim_max[TPW];
  bf16x8 qop[TPW][STEPS];
  float m_run[TPW], l_run[TPW];
  f32x4 l_acc[TPW];                                  // column sums in [0] (no page factors)
  f32x4 acc[TPW][DPL];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    r0[t] = (wave + NW * t) * unit;                  // the tile's first row in the block
    nqw[t] = max(0, min(unit, nq - r0[t]));          // its rows (uniform)
    const bool col_live = qr < nqw[t];
    lim[t] = col_live ? pos0 + r0[t] + qr : 0x7fffffff;
    lim_min[t] = pos0 + r0[t];
    lim_max[t] = pos0 + r0[t] + nqw[t] - 1;
    const int64_t qbase = ((int64_t)(qrow0 + r0[t] + qr) * a.n_q_heads + (int64_t)h * g + hh) * D;
#pragma unroll
    for (int s2 = 0; s2 < STEPS; ++s2) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col_live) v = *reinterpret_cast<const u32x4*>(a.q + qbase + 32 * s2 + 8 * kg);
      qop[t][s2] = __builtin_bit_cast(bf16x8, v);
    }
    m_run[t] = PAGE ? -INFINITY : -FLT_MAX;        // (the lazy reference of softmax_tiles)
    l_run[t] = 0.f;
    l_acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < DPL; ++nb) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int c_first = k0 / kChunk, c_last = (k1 - 1) / kChunk;
  const int n_st = (c_last - c_first) / SUB + 1;
  float cks[HALVES], cvs[HALVES];
  auto keep_factors = [&]() {
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf) {
      cks[hf] = ld.sks[hf];
      cvs[hf] = ld.svs[hf];
    }
  };
  __syncthreads();                  // the previous item's readers are done with buf
  ld.put(buf[0], tid);
  keep_factors();
  __syncthreads();
  for (int si = 0; si < n_st; ++si) {
    const int cur = si & 1;
    {
      // one call site, always issued (the waits before the stores then
      // count only its loads); after the last stage of the last item it
      // reloads this stage, which nothing stores
      const bool own = si + 1 < n_st;
      const bool nxt = !own && has_next;
      ld.fetch(a, block_table, nxt ? next_b : b, nxt ? next_L : L, h,
               own ? c_first + SUB * (si + 1) : nxt ? next_c : c_first + SUB * si, tid);
    }
    const SS& ss = buf[cur];
#pragma unroll
    for (int j = 0; j < SUB; ++j) {
      const int c = c_first + SUB * si + j;
      if (c > c_last) break;                          // uniform: the item's last stage
      // a tile whose columns see no token of this chunk skips its arithmetic
      // (and the wave its LDS reads when no tile needs them)
      bool need[TPW], any = false;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        need[t] = nqw[t] > 0 && c * kChunk <= lim_max[t];
        any = any || need[t];
      }
      if (!any) continue;
      // QK of every tile with rows (all products in flight before the first
      // softmax), the V operand reads, the softmax of every tile that sees
      // the chunk, then PV.  (With per-page factors, whose softmax holds more
      // registers, each tile's softmax follows its QK and the V reads come
      // after.)
      const float jks[2] = {cks[2 * j], cks[2 * j + 1]}, jvs[2] = {cvs[2 * j], cvs[2 * j + 1]};
      f32x4 sacc[TPW][2];
      bf16x8 pop[TPW];
      if constexpr (kHalves) {
        // fragments half by half (the register budget of four waves per
        // SIMD): K for 16 tokens, then their products
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          bf16x8 kh[STEPS];
#pragma unroll
          for (int s2 = 0; s2 < STEPS; ++s2)
            kh[s2] = *reinterpret_cast<const bf16x8*>(
                ss.k + SS::k_off(kChunk * j + 16 * hf + i, 4 * s2 + kg));
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            sacc[t][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < STEPS; ++s2)
              sacc[t][hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh[s2], qop[t][s2], sacc[t][hf], 0, 0, 0);
          }
        }
      } else {
        bf16x8 kf[2][STEPS];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int s2 = 0; s2 < STEPS; ++s2)
            kf[hf][s2] = *reinterpret_cast<const bf16x8*>(
                ss.k + SS::k_off(kChunk * j + 16 * hf + i, 4 * s2 + kg));
        // every fragment read in flight before the first product (left to
        // itself the scheduler can reuse one register set and wait on each
        // read in turn)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          if constexpr (!PAGE) {
            // every tile, branch-free (a tile without rows has q = 0)
            qk_scores<D>(kf, qop[t], sacc[t]);
          } else if (need[t]) {
            qk_scores<D>(kf, qop[t], sacc[t]);
            pop[t] = softmax_update<D / 16, true, true>(sacc[t], jks, jvs, c, k0, k1, lim[t],
                                                        lim_min[t], qk, kg, m_run[t], l_run[t],
                                                        acc[t]);
          }
        }
      }
      if constexpr (kHalves) {
        // the softmax, then V and its products half by half (dims blocks
        // 0..DPL/2-1, then the rest)
        softmax_tiles<D, TPW>(sacc, c, k0, k1, lim, lim_min, qk, kg, m_run, l_acc, acc, pop);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          bf16x8 vh[DPL / 2];
#pragma unroll
          for (int nb = 0; nb < DPL / 2; ++nb)
            vh[nb] = *reinterpret_cast<const bf16x8*>(ss.vt[j] + 1024 * (nb + DPL / 2 * h2) +
                                                       256 * kg + 16 * i);
#pragma unroll
          for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int nb = 0; nb < DPL / 2; ++nb)
              acc[t][nb + DPL / 2 * h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  vh[nb], pop[t], acc[t][nb + DPL / 2 * h2], 0, 0, 0);
        }
        continue;
      }
      bf16x8 vf[DPL];
#pragma unroll
      for (int nb = 0; nb < DPL; ++nb)
        vf[nb] = *reinterpret_cast<const bf16x8*>(ss.vt[j] + 1024 * nb + 256 * kg + 16 * i);
      if constexpr (!PAGE)
        softmax_tiles<D, TPW>(sacc, c, k0, k1, lim, lim_min, qk, kg, m_run, l_acc, acc, pop);
      __builtin_amdgcn_sched_barrier(0);
      // O^T block nb += V^T P^T; for bf16 pages without per-page factors for
      // every tile, branch-free (weights 0 where a tile sees none of the
      // chunk): measured faster there, slower for fp8 pages
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        if ((!PAGE && !FP8) || need[t])
#pragma unroll
          for (int nb = 0; nb < DPL; ++nb)
            acc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[nb], pop[t], acc[t][nb], 0, 0, 0);
    }
    if (si + 1 < n_st) {
      ld.put(buf[cur ^ 1], tid);
      keep_factors();
    }
    __syncthreads();
  }

  // finish the wave's own columns: lane (i, kg) holds column i, head dims
  // DPL * (4 kg + r) + nb in acc[nb][r] -- 4 DPL consecutive dims from
  // 4 DPL kg -- and a quarter of the column's weight sum
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    // (per-page factors: each lane holds a share of the column's sum)
    const float l_tot = PAGE ? kg_reduce_sum(l_run[t]) : l_acc[t][0];
    if (nqw[t] == 0) break;
    if (i < nqw[t] * g) {
      const int64_t hq = (int64_t)h * g + hh;
      const float inv = l_tot > 0.f ? vsc / l_tot : 0.f;
      float* dst;
      if (slot < 0)
        dst = a.out + ((int64_t)(qrow0 + r0[t] + qr) * a.n_q_heads + hq) * D;
      else
        dst = a.part_o + (((int64_t)slot * a.qb + r0[t] + qr) * a.n_q_heads + hq) * D;
      dst += 4 * DPL * kg;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int v4 = 0; v4 < DPL / 4; ++v4)
          *reinterpret_cast<f32x4*>(dst + DPL * r + 4 * v4) =
              f32x4{acc[t][4 * v4][r] * inv, acc[t][4 * v4 + 1][r] * inv,
                    acc[t][4 * v4 + 2][r] * inv, acc[t][4 * v4 + 3][r] * inv};
      if (slot >= 0 && kg == 0) {
        const int64_t prow = ((int64_t)slot * a.qb + r0[t] + qr) * a.n_q_heads + hq;
        a.part_lse[prow] = l_tot > 0.f ? (m_run[t] + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      }
    }
  }
}

template <int D, bool FP8, bool PAGE, int NW, int TPW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void hda_prefill_shared_kernel(
    Args a, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ plan) {
  __shared__ SharedStage<D, kSharedSub> buf[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % a.n_kv_heads;
  const int w = blockIdx.x / a.n_kv_heads;
  const int32_t* wg_ptr = plan + HDA_PLAN_HEADER_INTS;
  const int32_t* items = wg_ptr + a.n_wg + 1;
  const int32_t* __restrict__ rows = a.rows;
  const int it_begin = wg_ptr[w], it_end = wg_ptr[w + 1];
  auto well_formed = [&](int it) {
    const int rho = items[4 * it], k0 = items[4 * it + 1], k1 = items[4 * it + 2],
              slot = items[4 * it + 3];
    return (unsigned)rho < (unsigned)a.batch && k0 >= 0 && k1 > k0 && slot < a.n_parts;
  };
  // an item with tokens below its request's device length (the range is cut
  // there; see cut_at_len)
  auto valid = [&](int it) {
    return well_formed(it) &&
           min(items[4 * it + 2], seq_lens[rows[4 * items[4 * it]]]) > items[4 * it + 1];
  };
  auto next_valid = [&](int it) {
    while (it < it_end && !valid(it)) ++it;
    return it;
  };
  // Check bits; items left empty by the cut write an empty partial
  // (o = 0, lse = -inf: weighed zero by the merge) here, the others below.
  {
    const int g = a.group;
    int chk = 0;
    for (int it = it_begin; it < it_end; ++it) {
      if (!well_formed(it)) continue;
      const int rho = items[4 * it], k0 = items[4 * it + 1], slot = items[4 * it + 3];
      int k1 = items[4 * it + 2];
      chk |= cut_at_len(k1, seq_lens[rows[4 * rho]], false);
      if (k1 > k0 || slot < 0) continue;
      const int nq = rows[4 * rho + 2];
      for (int idx = tid; idx < nq * g * D; idx += 64 * NW) {
        const int r = idx / (g * D), rem = idx - r * g * D, hh = rem / D, d = rem - hh * D;
        const int64_t prow = ((int64_t)slot * a.qb + r) * a.n_q_heads + (int64_t)h * g + hh;
        a.part_o[prow * D + d] = 0.f;
        if (d == 0) a.part_lse[prow] = -INFINITY;
      }
    }
    write_check(a, chk, tid);
  }
  StageLoader<D, FP8, PAGE, NW, kSharedSub> ld;
  int it = next_valid(it_begin);
  if (it < it_end) {
    const int b = rows[4 * items[4 * it]];
    ld.fetch(a, block_table, b, seq_lens[b], h, items[4 * it + 1] / kChunk, tid);
  }
  while (it < it_end) {
    const int rho = items[4 * it], k0 = items[4 * it + 1], k1 = items[4 * it + 2],
              slot = items[4 * it + 3];
    const int b = rows[4 * rho], qrow0 = rows[4 * rho + 1], nq = rows[4 * rho + 2],
              pos0 = rows[4 * rho + 3];
    const int nx = next_valid(it + 1);
    const bool has_next = nx < it_end;
    const int next_b = has_next ? rows[4 * items[4 * nx]] : 0;
    const int next_L = has_next ? seq_lens[next_b] : 0;
    const int next_c = has_next ? items[4 * nx + 1] / kChunk : 0;
    const int L = seq_lens[b];
    process_item_shared<D, FP8, PAGE, NW, TPW, kSharedSub>(
        a, block_table, buf, ld, b, k0, min(k1, L), slot, L, qrow0, nq, pos0, h, has_next, next_b,
        next_L, next_c, wave, lane, tid);
    it = nx;
  }
}

// ---- device-side planning: the host planner's arithmetic, per wave ----
// T tiles over W workgroups, the first r = T mod W taking q + 1 tiles.
struct SplitDev {
  uint32_t q, r;
  __device__ uint32_t first_tile(uint32_t w) const { return w * q + min(w, r); }
  __device__ uint32_t owner(uint32_t t) const {
    const uint32_t big = r * (q + 1);
    return t < big ? t / (q + 1) : r + (t - big) / q;
  }
};

__device__ inline uint32_t tiles_of(int len, int tile_len) {
  return len > 0 ? (uint32_t)((len - 1) / tile_len + 1) : 0u;
}

__device__ inline uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ inline uint32_t wave_total_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Per-request plan facts for the 64 requests cb + lane, given the running
// totals over earlier requests: first tile, tile count, item count and the
// first partial slot.
struct ReqScan {
  int b, len;
  uint32_t n, first, k, slot_base;
};

__device__ inline ReqScan scan_requests(const int32_t* __restrict__ seq_lens, int batch,
                                        int tile_len, const SplitDev& sp, int cb, int lane,
                                        uint32_t first_carry, uint32_t slot_carry,
                                        uint32_t& first_total, uint32_t& split_total) {
  ReqScan r;
  r.b = cb + lane;
  r.len = r.b < batch ? seq_lens[r.b] : 0;
  r.n = tiles_of(r.len, tile_len);
  const uint32_t incl = wave_incl_scan(r.n, lane);
  r.first = first_carry + incl - r.n;
  r.k = r.n ? sp.owner(r.first + r.n - 1) - sp.owner(r.first) + 1 : 0u;
  const uint32_t split_k = r.k > 1 ? r.k : 0u;
  const uint32_t sincl = wave_incl_scan(split_k, lane);
  r.slot_base = slot_carry + sincl - split_k;
  first_total = __shfl(incl, 63);
  split_total = __shfl(sincl, 63);
  return r;
}

__device__ inline uint32_t total_tiles(const int32_t* __restrict__ seq_lens, int batch,
                                       int tile_len, int lane) {
  uint32_t T = 0;
  for (int cb = 0; cb < batch; cb += 64) {
    const int b = cb + lane;
    T += wave_total_u32(b < batch ? tiles_of(seq_lens[b], tile_len) : 0u);
  }
  return __builtin_amdgcn_readfirstlane(T);
}

// One item by the kernel variant's item routine.
template <int D, bool FP8, bool PAGE, bool NATIVE, bool COVER = false>
__device__ inline void run_item(const Args& a, const int32_t* __restrict__ block_table,
                                TileSmem<D>& sm, int b, int k0, int k1, int slot, int L, int h,
                                int wave, int lane, int tid) {
  if constexpr (NATIVE)
    process_item_fp8n<COVER>(a, block_table, sm, b, k0, k1, slot, L, h, wave, lane, tid);
  else
    process_item<D, FP8, PAGE, false, COVER>(a, block_table, sm, b, k0, k1, slot, L, b, 1, L - 1,
                                             h, wave, lane, tid);
}


// Workgroup (w, h): W * Hkv workgroups, kv head fastest.  Items come from the
// host plan (DEVPLAN false) or are derived here from the device lengths with
// the same rule (DEVPLAN true), in the same order.  NATIVE selects the
// native-fp8 item routine (D = 128).
template <int D, bool FP8, bool DEVPLAN, bool PAGE, bool NATIVE, bool PF = false,
          bool COVER = false>
__global__ __launch_bounds__(64 * kWaves, 2) void hda_decode_kernel(
    Args a, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ plan) {
  // The plan, lengths and block table are read-only here and reached by
  // wave-uniform addresses, so they load through the scalar cache.
  __shared__ TileSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index is uniform within a wave: keep it (and everything derived
  // from it: chunk index, page id, buffer resources) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % a.n_kv_heads;
  const int w = blockIdx.x / a.n_kv_heads;

  if constexpr (PF) {
    // multi-token rows: a plan "request" is a row block
    const int32_t* wg_ptr = plan + HDA_PLAN_HEADER_INTS;
    const int32_t* items = wg_ptr + a.n_wg + 1;
    const int it_begin = wg_ptr[w], it_end = wg_ptr[w + 1];
    const int32_t* __restrict__ rows = a.rows;
    int chk = 0;
    for (int it = it_begin; it < it_end; ++it) {
      const int rho = items[4 * it], k0 = items[4 * it + 1], slot = items[4 * it + 3];
      int k1 = items[4 * it + 2];
      if ((unsigned)rho >= (unsigned)a.batch || k0 < 0 || k1 <= k0 || slot >= a.n_parts) continue;
      const int b = rows[4 * rho], qrow0 = rows[4 * rho + 1], nq = rows[4 * rho + 2],
                pos0 = rows[4 * rho + 3];
      const int L = seq_lens[b];
      chk |= cut_at_len(k1, L, false);
      process_item<D, FP8, PAGE, true>(a, block_table, sm, b, k0, k1, slot, L, qrow0, nq, pos0, h,
                                       wave, lane, tid);
    }
    write_check(a, chk, tid);
  } else if constexpr (!DEVPLAN) {
    const int32_t* wg_ptr = plan + HDA_PLAN_HEADER_INTS;
    const int32_t* items = wg_ptr + a.n_wg + 1;
    const int it_begin = wg_ptr[w], it_end = wg_ptr[w + 1];
    int chk = 0;
    for (int it = it_begin; it < it_end; ++it) {
      const int b = items[4 * it], k0 = items[4 * it + 1], slot = items[4 * it + 3];
      int k1 = items[4 * it + 2];
      if ((unsigned)b >= (unsigned)a.batch || k0 < 0 || k1 <= k0 || slot >= a.n_parts) continue;
      const int L = seq_lens[b];
      chk |= cut_at_len(k1, L, it + 1 >= a.n_items || items[4 * (it + 1)] != b);
      run_item<D, FP8, PAGE, NATIVE, COVER>(a, block_table, sm, b, k0, k1, slot, L, h, wave, lane,
                                            tid);
    }
    write_check(a, chk, tid);
  } else {
    // the plan comes from the device lengths themselves: nothing to check
    write_check(a, 0, tid);
    // Every wave derives the same plan facts; they stay wave-uniform.
    const uint32_t T = total_tiles(seq_lens, a.batch, a.tile_len, lane);
    const SplitDev sp{T / (uint32_t)a.n_wg, T % (uint32_t)a.n_wg};
    const uint32_t t0 = sp.first_tile(w), t1 = sp.first_tile(w + 1);
    if (t0 >= t1) return;
    uint32_t first_carry = 0, slot_carry = 0;
    for (int cb = 0; cb < a.batch && first_carry < t1; cb += 64) {
      uint32_t ft, st;
      const ReqScan r = scan_requests(seq_lens, a.batch, a.tile_len, sp, cb, lane, first_carry,
                                      slot_carry, ft, st);
      // the workgroup holding a request's first tile records its slot range
      // for the merge launch (kv head 0 only; every head would write the same)
      if (h == 0 && r.n > 0 && r.first >= t0 && r.first < t1) {
        a.req_slots[2 * r.b] = (int32_t)r.slot_base;
        a.req_slots[2 * r.b + 1] = r.k > 1 ? (int32_t)r.k : 0;
      }
      uint64_t mask = __ballot(r.n > 0 && r.first < t1 && r.first + r.n > t0);
      while (mask) {
        const int j = __builtin_ctzll(mask);
        mask &= mask - 1;
        const int b = __builtin_amdgcn_readlane(r.b, j);
        const int L = __builtin_amdgcn_readlane(r.len, j);
        const uint32_t first = __builtin_amdgcn_readlane(r.first, j);
        const uint32_t n = __builtin_amdgcn_readlane(r.n, j);
        const uint32_t k = __builtin_amdgcn_readlane(r.k, j);
        const uint32_t sb = __builtin_amdgcn_readlane(r.slot_base, j);
        const uint32_t lo = max(t0, first), hi = min(t1, first + n);
        const int k0 = (int)((int64_t)(lo - first) * a.tile_len);
        const int k1 = (int)min((int64_t)(hi - first) * a.tile_len, (int64_t)L);
        const int slot = k > 1 ? (int)(sb + (uint32_t)w - sp.owner(first)) : -1;
        run_item<D, FP8, PAGE, NATIVE>(a, block_table, sm, b, k0, k1, slot, L, h, wave, lane,
                                       tid);
      }
      first_carry += ft;
      slot_carry += st;
    }
  }
}

// The same tile kernel for a host plan carried in the launch arguments (at
// most kArgPlanInts ints): no upload precedes it on the stream.  Workgroup 0
// also turns req_part_ptr into the per-request slot ranges the merge launch
// reads, as a device-planned launch records them.
constexpr int kArgPlanInts = HDA_PLAN_ARG_INTS;
struct ArgPlan {
  int32_t v[kArgPlanInts];
};

template <int D, bool FP8, bool PAGE, bool NATIVE>
__global__ __launch_bounds__(64 * kWaves, 2) void hda_decode_argplan_kernel(
    Args a, const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    ArgPlan pl) {
  __shared__ TileSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.x % a.n_kv_heads;
  const int w = blockIdx.x / a.n_kv_heads;
  const int32_t* wg_ptr = pl.v + HDA_PLAN_HEADER_INTS;
  const int32_t* items = wg_ptr + a.n_wg + 1;
  if (a.n_parts > 0 && a.req_slots && blockIdx.x == 0) {   // (a merge list needs none)
    const int32_t* rpp = items + 4 * a.n_items;
    for (int b = tid; b < a.batch; b += 64 * kWaves) {
      const int s0 = rpp[b];
      a.req_slots[2 * b] = s0;
      a.req_slots[2 * b + 1] = rpp[b + 1] - s0;
    }
  }
  const int it_begin = wg_ptr[w], it_end = wg_ptr[w + 1];
  int chk = 0;
  for (int it = it_begin; it < it_end; ++it) {
    const int b = items[4 * it], k0 = items[4 * it + 1], slot = items[4 * it + 3];
    int k1 = items[4 * it + 2];
    if ((unsigned)b >= (unsigned)a.batch || k0 < 0 || k1 <= k0 || slot >= a.n_parts) continue;
    const int L = seq_lens[b];
    chk |= cut_at_len(k1, L, it + 1 >= a.n_items || items[4 * (it + 1)] != b);
    run_item<D, FP8, PAGE, NATIVE>(a, block_table, sm, b, k0, k1, slot, L, h, wave, lane, tid);
  }
  write_check(a, chk, tid);
}

// Log-sum-exp merge of split requests: workgroup (b, q head) combines the
// partials of request b in slot order,
//   out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M),  M = max_s lse_s.
// A separate launch: the kernel boundary makes every partial written by the
// tile kernel (on any XCD) visible here without cross-XCD fences.  Thread d
// owns output dim d.  The first kMergeEarly partial rows are loaded up front,
// before the weights are known, so that the whole merge costs about one
// memory round trip for typical slot counts.  (One workgroup per kv head
// instead was measured 3x slower on a request split 32 ways.)  RECORDED: the
// slot ranges come from a.req_slots, where the tile kernel recorded them (a
// device-planned launch, or a plan in the launch arguments), else from the
// plan's req_part_ptr in device memory.
constexpr int kMergeEarly = 32;    // partial rows loaded before the weights
constexpr int kMergeStage = 512;   // slot weights staged in LDS per pass

// Where the merge finds each request's slot range: the plan's req_part_ptr
// in device memory, the ranges the tile kernel recorded in the workspace,
// or a list of the split requests in the merge's own launch arguments (the
// host knows them from its plan; the grid then covers only those requests).
// (Plain int constants, not an enum: a kernel's mangled name must come out
// the same in the host and the device compilation, and an unnamed type's
// compiler-made name need not.)
constexpr int kSlotsPlan = 0, kSlotsRecorded = 1, kSlotsList = 2;
constexpr int kMergeListMax = 256;
struct MergeList {
  int32_t v[3 * kMergeListMax];   // (request, first slot, slot count) per split request
};
struct NoMergeList {};
template <int SRC>
using MergeArg = typename std::conditional<SRC == kSlotsList, MergeList, NoMergeList>::type;

template <int D, int SRC>
__global__ __launch_bounds__(D) void hda_merge_kernel(Args a, const int32_t* __restrict__ plan,
                                                      const int32_t* __restrict__ seq_lens,
                                                      MergeArg<SRC> ml) {
  __shared__ float sm_w[kMergeStage];
  __shared__ float sm_red[2][D / 64];
  const int d = threadIdx.x, lane = d & 63, wave = d >> 6;
  const int hq = blockIdx.x % a.n_q_heads;
  const int e = blockIdx.x / a.n_q_heads;
  const int qr = 0;
  int b, s0, s1;
  if constexpr (SRC == kSlotsList) {
    b = ml.v[3 * e];
    s0 = max(0, ml.v[3 * e + 1]);
    s1 = min(a.n_parts, ml.v[3 * e + 1] + ml.v[3 * e + 2]);
  } else if constexpr (SRC == kSlotsPlan) {
    b = e;
    const int32_t* rpp = plan + HDA_PLAN_HEADER_INTS + a.n_wg + 1 + 4 * a.n_items;
    s0 = max(0, rpp[b]);
    s1 = min(a.n_parts, rpp[b + 1]);
  } else {
    b = e;
    if (seq_lens[b] < 1) return;                    // no item, nothing recorded
    s0 = max(0, a.req_slots[2 * b]);
    s1 = min(a.n_parts, s0 + a.req_slots[2 * b + 1]);
  }
  const int orow = b;
  if (s1 <= s0) return;
  const int n = s1 - s0;
  const int64_t lstride = (int64_t)a.qb * a.n_q_heads;   // between slots, in rows
  const int64_t row_stride = lstride * D;
  const float* po = a.part_o + ((int64_t)s0 * lstride + (int64_t)qr * a.n_q_heads + hq) * D + d;
  const float* lse = a.part_lse + (int64_t)s0 * lstride + (int64_t)qr * a.n_q_heads + hq;

  float early[kMergeEarly];
#pragma unroll
  for (int u = 0; u < kMergeEarly; ++u) early[u] = u < n ? po[(int64_t)u * row_stride] : 0.f;
  float my_lse = d < n ? lse[(int64_t)d * lstride] : -INFINITY;

  float m = my_lse;
  for (int k = d + D; k < n; k += D) m = fmaxf(m, lse[(int64_t)k * lstride]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) sm_red[0][wave] = m;
  __syncthreads();
  float M = sm_red[0][0];
#pragma unroll
  for (int w = 1; w < D / 64; ++w) M = fmaxf(M, sm_red[0][w]);
  float t = d < n ? expf(my_lse - M) : 0.f;
  for (int k = d + D; k < n; k += D) t += expf(lse[(int64_t)k * lstride] - M);
  t = wave_sum(t);
  if (lane == 0) sm_red[1][wave] = t;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < D / 64; ++w) total += sm_red[1][w];
  const float inv_total = 1.0f / total;

  float acc = 0.f;
  for (int c0 = 0; c0 < n; c0 += kMergeStage) {
    const int cn = min(kMergeStage, n - c0);
    if (c0 > 0) __syncthreads();
    for (int k = d; k < cn; k += D) {
      const float l = (c0 == 0 && k == d) ? my_lse : lse[(int64_t)(c0 + k) * lstride];
      sm_w[k] = expf(l - M) * inv_total;
    }
    __syncthreads();
    int k = 0;
    if (c0 == 0) {
#pragma unroll
      for (int u = 0; u < kMergeEarly; ++u)
        if (u < cn) acc += sm_w[u] * early[u];
      k = kMergeEarly;
    }
    for (; k + 16 <= cn; k += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = po[(int64_t)(c0 + k + u) * row_stride];
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += sm_w[k + u] * v[u];
    }
    for (; k < cn; ++k) acc += sm_w[k] * po[(int64_t)(c0 + k) * row_stride];
  }
  a.out[((int64_t)orow * a.n_q_heads + hq) * D + d] = acc;
}

// Merge of multi-token partials: workgroup (row block, row in block, group
// of 256 / (D/4) q heads), 256 threads, thread t owning float4 column t % Q
// (Q = D/4) of head t / Q of the group.  Per head, the weights are the
// decode merge's, computed in the same order (max over slots; the sum of
// exp(lse - M) as the decode merge's D/64 waves would add it, each wave's
// lanes taking slots lane + 64w, + D, ... and reducing with the same
// butterfly; the slots accumulated in order), so a row merges to exactly
// what hda_merge_kernel gives.  The first 16 slots' outputs are loaded before
// the weights are known, then eight slots' loads at a time.  (One workgroup of D threads per row and head
// measured latency-bound on multi-token batches: 2.2x slower.)
constexpr int kMergeRowsThreads = 256;

template <int D, int E>
__global__ __launch_bounds__(kMergeRowsThreads) void hda_merge_rows_kernel(
    Args a, const int32_t* __restrict__ plan) {
  constexpr int Q = D / 4;                           // float4 columns per head
  constexpr int HPW = kMergeRowsThreads / Q;         // heads per workgroup
  constexpr int NWV = kMergeRowsThreads / 64;        // waves
  constexpr int HPV = (HPW + NWV - 1) / NWV;         // heads per wave in the weight pass
  constexpr int U = 8;                               // slots in flight past the first E
  // E: slots loaded before the weights (the launch picks the smallest of 2,
  // 4, 8, 16 that holds the plan's largest slot count, up to 16: the loads
  // are clamped, not branched, so every early load is issued)
  __shared__ float sM[HPW], sInv[HPW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Hq = a.n_q_heads;
  const int groups = (Hq + HPW - 1) / HPW;
  const int rb = blockIdx.x / groups, hg = blockIdx.x - rb * groups;
  const int b = rb / a.qb, qr = rb - b * a.qb;
  const int32_t* __restrict__ rows = a.rows;
  if (qr >= rows[4 * b + 2]) return;                // past the block's rows
  const int orow = rows[4 * b + 1] + qr;
  const int32_t* rpp = plan + HDA_PLAN_HEADER_INTS + a.n_wg + 1 + 4 * a.n_items;
  const int s0 = max(0, rpp[b]), s1 = min(a.n_parts, rpp[b + 1]);
  if (s1 <= s0) return;
  const int n = s1 - s0;
  const int64_t lstride = (int64_t)a.qb * Hq;       // between slots, in rows
  const float* lse = a.part_lse + (int64_t)s0 * lstride + (int64_t)qr * Hq;
  const int j = tid / Q, h = hg * HPW + j;           // this thread's head in the output pass
  const int hc = min(h, Hq - 1);                     // loads stay in range past Hq
  const int64_t row_stride = lstride * D;            // floats between slots
  const float* po = a.part_o + ((int64_t)s0 * lstride + (int64_t)qr * Hq + hc) * D + 4 * (tid % Q);
  const float* lh = lse + hc;
  // Loads in issue order: the weight pass's lse values (slot = lane), then
  // the first E slots' outputs and lse for the output pass.  Completion
  // counting is in order, so the weight pass waits for its own loads only.
  // Indices are clamped rather than branched around, so no wait is merged.
  float ls[HPV];
#pragma unroll
  for (int jj = 0; jj < HPV; ++jj) {
    const int hw = min(hg * HPW + wave + NWV * jj, Hq - 1);
    ls[jj] = lse[(int64_t)min(lane, n - 1) * lstride + hw];
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 v0[E];
  float l0[E];
#pragma unroll
  for (int u = 0; u < E; ++u) {
    const int64_t k = min(u, n - 1);
    v0[u] = *reinterpret_cast<const f32x4*>(po + k * row_stride);
    l0[u] = lh[k * lstride];
  }
  __builtin_amdgcn_sched_barrier(0);
  // weights per head: max over slots, then the sum of exp(lse - M) as the
  // decode merge's D/64 waves add it (lanes take slots lane + 64w, + D, ...);
  // slot `lane` comes from ls, further slots (n > 64) are loaded here
  float mh[HPV];
#pragma unroll
  for (int jj = 0; jj < HPV; ++jj) mh[jj] = lane < n ? fmaxf(-INFINITY, ls[jj]) : -INFINITY;
  if (n > 64) {
#pragma unroll
    for (int jj = 0; jj < HPV; ++jj) {
      const int hw = min(hg * HPW + wave + NWV * jj, Hq - 1);
      for (int k = lane + 64; k < n; k += 64) mh[jj] = fmaxf(mh[jj], lse[(int64_t)k * lstride + hw]);
    }
  }
#pragma unroll
  for (int jj = 0; jj < HPV; ++jj) {
    const int jw = wave + NWV * jj;
    const int hw = min(hg * HPW + jw, Hq - 1);
    float m = mh[jj];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float total = wave_sum(lane < n ? expf(ls[jj] - m) : 0.f);
    if (n > 64) {
      total = 0.f;
#pragma unroll
      for (int w = 0; w < D / 64; ++w) {
        const int d = 64 * w + lane;
        float t = d < n ? expf(lse[(int64_t)d * lstride + hw] - m) : 0.f;
        for (int k = d + D; k < n; k += D) t += expf(lse[(int64_t)k * lstride + hw] - m);
        total += wave_sum(t);
      }
    }
    if (lane == 0 && jw < HPW && hg * HPW + jw < Hq) {
      sM[jw] = m;
      sInv[jw] = 1.0f / total;
    }
  }
  // LDS-only barrier: the output loads above stay in flight across it
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  if (h >= Hq) return;
  const float M = sM[j], inv = sInv[j];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < E; ++u) {
    if (u < n) {
      const float w = expf(l0[u] - M) * inv;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += w * v0[u][e];
    }
  }
  int k = E;
  for (; k + U <= n; k += U) {
    f32x4 v[U];
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)(k + u) * row_stride);
      l[u] = lh[(int64_t)(k + u) * lstride];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = expf(l[u] - M) * inv;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += w * v[u][e];
    }
  }
  for (; k < n; ++k) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(po + (int64_t)k * row_stride);
    const float w = expf(lh[(int64_t)k * lstride] - M) * inv;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += w * v[e];
  }
  *reinterpret_cast<f32x4*>(a.out + ((int64_t)orow * Hq + h) * D + 4 * (tid % Q)) = acc;
}

// A host plan carried to device memory inside a launch's kernel arguments:
// the runtime copies the arguments when the launch is enqueued, so the
// stream sees one small kernel and no separate copy, and the caller's host
// buffer is free again as soon as the launch returns.
constexpr int kUploadInts = HDA_PLAN_UPLOAD_CHUNK;
struct UploadChunk {
  int32_t v[kUploadInts];
};

static_assert(kUploadInts <= 4 * 256, "one load round per thread");

__global__ __launch_bounds__(256) void hda_plan_store_kernel(UploadChunk c,
                                                             int32_t* __restrict__ dst, int n) {
  int32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // all argument reads in flight before the stores
    const int i = threadIdx.x + 256 * j;
    r[j] = i < n ? c.v[i] : 0;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < n) dst[i] = r[j];
  }
}

// The plan in the host format, built from device lengths by one wave with
// the device-side planning arithmetic (the same items the tile kernel derives
// for itself in a device-planned launch).
__global__ __launch_bounds__(64) void hda_plan_kernel(const int32_t* __restrict__ seq_lens,
                                                      int batch, int tile_len, int W,
                                                      int32_t* __restrict__ plan) {
  const int lane = threadIdx.x;
  const uint32_t T = total_tiles(seq_lens, batch, tile_len, lane);
  const SplitDev sp{T / (uint32_t)W, T % (uint32_t)W};
  int32_t* wg_ptr = plan + HDA_PLAN_HEADER_INTS;
  int32_t* items = wg_ptr + W + 1;
  // pass 1: item count N (items sit between wg_ptr and req_part_ptr)
  uint32_t N = 0, P = 0;
  {
    uint32_t fc = 0, sc = 0;
    for (int cb = 0; cb < batch; cb += 64) {
      uint32_t ft, st;
      const ReqScan r = scan_requests(seq_lens, batch, tile_len, sp, cb, lane, fc, sc, ft, st);
      N += wave_total_u32(r.k);
      fc += ft;
      sc += st;
    }
    P = sc;
  }
  int32_t* rpp = items + 4 * N;
  // pass 2: items, req_part_ptr, and wg_ptr contributions
  uint32_t fc = 0, sc = 0, ic = 0;
  for (int cb = 0; cb < batch; cb += 64) {
    uint32_t ft, st;
    const ReqScan r = scan_requests(seq_lens, batch, tile_len, sp, cb, lane, fc, sc, ft, st);
    const uint32_t iincl = wave_incl_scan(r.k, lane);
    const uint32_t ibase = ic + iincl - r.k;
    if (r.b < batch) {
      const uint32_t w0 = r.n ? sp.owner(r.first) : 0u;
      for (uint32_t j = 0; j < r.k; ++j) {
        const uint32_t wg = w0 + j;
        const uint32_t lo = max(r.first, sp.first_tile(wg));
        const uint32_t hi = min(r.first + r.n, sp.first_tile(wg + 1));
        int32_t* it = items + 4 * (ibase + j);
        it[0] = r.b;
        it[1] = (int32_t)((int64_t)(lo - r.first) * tile_len);
        it[2] = (int32_t)min((int64_t)(hi - r.first) * tile_len, (int64_t)r.len);
        it[3] = r.k > 1 ? (int32_t)(r.slot_base + j) : -1;
      }
      rpp[r.b + 1] = (int32_t)(r.slot_base + (r.k > 1 ? r.k : 0u));
    }
    fc += ft;
    sc += st;
    ic += __shfl(iincl, 63);
  }
  // wg_ptr[w] = number of items held by workgroups before w
  for (int w = 0; w <= W; ++w) {
    uint32_t cnt = 0, fc2 = 0, sc2 = 0;
    for (int cb = 0; cb < batch; cb += 64) {
      uint32_t ft, st;
      const ReqScan r = scan_requests(seq_lens, batch, tile_len, sp, cb, lane, fc2, sc2, ft, st);
      uint32_t c = 0;
      if (r.k) {
        const uint32_t w0 = sp.owner(r.first);
        c = (uint32_t)w > w0 ? min((uint32_t)w - w0, r.k) : 0u;
      }
      cnt += wave_total_u32(c);
      fc2 += ft;
      sc2 += st;
    }
    if (lane == 0) wg_ptr[w] = (int32_t)cnt;
  }
  if (lane == 0) {
    rpp[0] = 0;
    plan[0] = HDA_PLAN_VERSION;
    plan[1] = batch;
    plan[2] = tile_len;
    plan[3] = W;
    plan[4] = (int32_t)T;
    plan[5] = (int32_t)N;
    plan[6] = (int32_t)P;
    plan[7] = 0;
  }
}

template <int D, bool FP8, bool DEVPLAN, bool PAGE, bool NATIVE = false, bool COVER = false>
hipError_t launch(Args a, int grid, bool prologue, uint16_t* q_prime, hipStream_t stream,
                  void* split_event, const ArgPlan* ap, const MergeList* ml, int n_split) {
  if (ml) a.req_slots = nullptr;   // the merge's ranges travel in its own arguments
  hipError_t e;
  if (prologue) {
    hipLaunchKernelGGL((hda_prologue_kernel<D, FP8>), dim3(a.batch * a.n_kv_heads), dim3(256), 0,
                       stream, a, a.block_table, a.seq_lens, q_prime);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.q = q_prime;   // attention reads the normalised, rotated q
  }
  if (!DEVPLAN && ap)
    hipLaunchKernelGGL((hda_decode_argplan_kernel<D, FP8, PAGE, NATIVE>), dim3(grid),
                       dim3(64 * kWaves), 0, stream, a, a.block_table, a.seq_lens, *ap);
  else
    hipLaunchKernelGGL((hda_decode_kernel<D, FP8, DEVPLAN, PAGE, NATIVE, false, COVER>),
                       dim3(grid), dim3(64 * kWaves), 0, stream, a, a.block_table, a.seq_lens,
                       a.plan);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (split_event) {
    e = hipEventRecord(static_cast<hipEvent_t>(split_event), stream);
    if (e != hipSuccess) return e;
  }
  if (DEVPLAN || a.n_parts > 0) {
    // slot ranges from the host's list of split requests, else recorded by
    // the tile kernel (device plan, argument plan), else from plan_dev
    if (!DEVPLAN && ml)
      hipLaunchKernelGGL((hda_merge_kernel<D, kSlotsList>), dim3(n_split * a.n_q_heads), dim3(D),
                         0, stream, a, a.plan, a.seq_lens, *ml);
    else if (DEVPLAN || ap)
      hipLaunchKernelGGL((hda_merge_kernel<D, kSlotsRecorded>), dim3(a.batch * a.n_q_heads),
                         dim3(D), 0, stream, a, a.plan, a.seq_lens, NoMergeList{});
    else
      hipLaunchKernelGGL((hda_merge_kernel<D, kSlotsPlan>), dim3(a.batch * a.n_q_heads), dim3(D),
                         0, stream, a, a.plan, a.seq_lens, NoMergeList{});
    e = hipGetLastError();
  }
  return e;
}

static_assert(HDA_PREFILL_MAX_TILES == 16, "largest block: 8 waves of two tiles");

template <int D, bool FP8, bool PAGE>
hipError_t launch_prefill(Args a, int grid, int n_rows, int max_slots, hipStream_t stream,
                          void* split_event) {
  // by the largest block, in tiles of 16/g rows: one tile on the decode
  // kernel's column shape (the waves split the item's chunks), else chunks
  // shared through LDS by 4 waves of one tile, 8 waves of one, or for the
  // largest blocks 8 waves of two -- 16 waves of one for an fp8 cache
  // without per-page factors, whose stage stores decode the codes (the
  // extra waves hide that work: 641 -> 607 us on the chunked fp8 mix; 602 ->
  // 631 us for bf16, which keeps 8 x 2)
  const int unit = kMaxGroup / a.group;
  const dim3 blk(64 * kWaves);
  if (a.qb <= unit)
    hipLaunchKernelGGL((hda_decode_kernel<D, FP8, false, PAGE, false, true>), dim3(grid), blk, 0,
                       stream, a, a.block_table, a.seq_lens, a.plan);
  else if (a.qb <= 4 * unit)
    hipLaunchKernelGGL((hda_prefill_shared_kernel<D, FP8, PAGE, 4, 1>), dim3(grid), blk, 0, stream,
                       a, a.block_table, a.seq_lens, a.plan);
  else if (a.qb <= 8 * unit)
    hipLaunchKernelGGL((hda_prefill_shared_kernel<D, FP8, PAGE, 8, 1>), dim3(grid), dim3(512), 0,
                       stream, a, a.block_table, a.seq_lens, a.plan);
  else if constexpr (FP8 && !PAGE)
    hipLaunchKernelGGL((hda_prefill_shared_kernel<D, FP8, PAGE, 16, 1>), dim3(grid), dim3(1024),
                       0, stream, a, a.block_table, a.seq_lens, a.plan);
  else
    hipLaunchKernelGGL((hda_prefill_shared_kernel<D, FP8, PAGE, 8, 2>), dim3(grid), dim3(512), 0,
                       stream, a, a.block_table, a.seq_lens, a.plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (split_event) {
    e = hipEventRecord(static_cast<hipEvent_t>(split_event), stream);
    if (e != hipSuccess) return e;
  }
  if (a.n_parts == 0) return e;
  const int groups = (a.n_q_heads + kMergeRowsThreads / (D / 4) - 1) / (kMergeRowsThreads / (D / 4));
  const dim3 mgrid(n_rows * a.qb * groups), mblk(kMergeRowsThreads);
  if (max_slots <= 2)
    hipLaunchKernelGGL((hda_merge_rows_kernel<D, 2>), mgrid, mblk, 0, stream, a, a.plan);
  else if (max_slots <= 4)
    hipLaunchKernelGGL((hda_merge_rows_kernel<D, 4>), mgrid, mblk, 0, stream, a, a.plan);
  else if (max_slots <= 8)
    hipLaunchKernelGGL((hda_merge_rows_kernel<D, 8>), mgrid, mblk, 0, stream, a, a.plan);
  else
    hipLaunchKernelGGL((hda_merge_rows_kernel<D, 16>), mgrid, mblk, 0, stream, a, a.plan);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const Args& a, bool fp8, int grid, int n_rows, int max_slots,
                            hipStream_t st, void* ev) {
  if (!fp8) return launch_prefill<D, false, false>(a, grid, n_rows, max_slots, st, ev);
  return a.scale_mode == HDA_SCALE_PAGE
             ? launch_prefill<D, true, true>(a, grid, n_rows, max_slots, st, ev)
             : launch_prefill<D, true, false>(a, grid, n_rows, max_slots, st, ev);
}

// Per-page scales are built for the fp8 cache only (check_params refuses
// them for bf16).
template <int D, bool DEVPLAN, bool COVER = false>
hipError_t launch_d(const Args& a, bool fp8, bool native, int grid, bool pro, uint16_t* qp,
                    hipStream_t st, void* ev, const ArgPlan* ap = nullptr,
                    const MergeList* ml = nullptr, int ns = 0) {
  if constexpr (D == 128)
    if (native)
      return launch<128, true, DEVPLAN, false, true, COVER>(a, grid, pro, qp, st, ev, ap, ml, ns);
  if (!fp8)
    return launch<D, false, DEVPLAN, false, false, COVER>(a, grid, pro, qp, st, ev, ap, ml, ns);
  return a.scale_mode == HDA_SCALE_PAGE
             ? launch<D, true, DEVPLAN, true, false, COVER>(a, grid, pro, qp, st, ev, ap, ml, ns)
             : launch<D, true, DEVPLAN, false, false, COVER>(a, grid, pro, qp, st, ev, ap, ml, ns);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Checks shared by both decode entry points (host only, before any launch).
int check_params(const hda_params* p, const void* q, const void* k_pages, const void* v_pages,
                 const void* block_table, const void* seq_lens, const void* out) {
  if (!p || !q || !k_pages || !v_pages || !block_table || !seq_lens || !out)
    return HDA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1 || p->head_dim < 1 ||
      p->page_size < 1 || p->max_pages_per_req < 1 || p->num_pages < 1)
    return HDA_ERR_INVALID_ARG;
  if (!(p->sm_scale > 0.f) || !(p->k_scale > 0.f) || !(p->v_scale > 0.f) ||
      !isfinite(p->sm_scale) || !isfinite(p->k_scale) || !isfinite(p->v_scale))
    return HDA_ERR_INVALID_ARG;
  if (p->n_q_heads % p->n_kv_heads != 0) return HDA_ERR_INVALID_ARG;
  if (p->n_q_heads / p->n_kv_heads > kMaxGroup) return HDA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return HDA_ERR_UNSUPPORTED;
  if (p->page_size < 16 || p->page_size > 1024 || (p->page_size & (p->page_size - 1)))
    return HDA_ERR_UNSUPPORTED;
  if (p->kv_dtype != HDA_KV_BF16 && p->kv_dtype != HDA_KV_FP8_E4M3) return HDA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages)) return HDA_ERR_INVALID_ARG;
  if (p->prologue) {
    if (!p->q_norm_w || !p->k_norm_w || !p->k_new || !p->v_new) return HDA_ERR_INVALID_ARG;
    if (!(p->rms_eps >= 0.f) || !(p->rope_theta > 0.f)) return HDA_ERR_INVALID_ARG;
  }
  if (p->scale_mode != HDA_SCALE_TENSOR && p->scale_mode != HDA_SCALE_HEAD &&
      p->scale_mode != HDA_SCALE_PAGE)
    return HDA_ERR_INVALID_ARG;
  if (p->scale_mode != HDA_SCALE_TENSOR && (!p->k_scales || !p->v_scales))
    return HDA_ERR_INVALID_ARG;
  if (p->scale_mode == HDA_SCALE_PAGE && p->kv_dtype != HDA_KV_FP8_E4M3) return HDA_ERR_UNSUPPORTED;
  if (p->math != HDA_MATH_BF16 && p->math != HDA_MATH_FP8) return HDA_ERR_INVALID_ARG;
  if (p->v_layout != HDA_V_TOKEN_MAJOR && p->v_layout != HDA_V_DIM_MAJOR) return HDA_ERR_INVALID_ARG;
  if (p->reserved0 != 0) return HDA_ERR_INVALID_ARG;
  // the native-fp8 kernel: fp8 cache, dim-major V, D 128, pages of >= 64
  // tokens, tensor or head scales; dim-major V pages only with it
  if (p->math == HDA_MATH_FP8 &&
      (p->kv_dtype != HDA_KV_FP8_E4M3 || p->v_layout != HDA_V_DIM_MAJOR || p->head_dim != 128 ||
       p->page_size < 64 || p->scale_mode == HDA_SCALE_PAGE))
    return HDA_ERR_UNSUPPORTED;
  if (p->v_layout == HDA_V_DIM_MAJOR && p->math != HDA_MATH_FP8) return HDA_ERR_UNSUPPORTED;
  return HDA_OK;
}

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// Workgroup item ranges of a plan (header and length already checked):
// wg_ptr from 0, non-decreasing, ending at N, so that the kernels' item
// loops stay inside the item list (the items themselves are range-checked
// on the device).
bool wg_ranges_ok(const int32_t* plan, int64_t W, int64_t N) {
  const int32_t* wg_ptr = plan + HDA_PLAN_HEADER_INTS;
  if (wg_ptr[0] != 0 || wg_ptr[W] != N) return false;
  for (int64_t w = 0; w < W; ++w)
    if (wg_ptr[w + 1] < wg_ptr[w]) return false;
  return true;
}

Args make_args(const hda_params* p, const void* q, void* k_pages, void* v_pages,
               const int32_t* block_table, const int32_t* seq_lens, float* out, int64_t W,
               int64_t P) {
  const int D = p->head_dim;
  const int elem = p->kv_dtype == HDA_KV_FP8_E4M3 ? 1 : 2;
  Args a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_pages = static_cast<uint8_t*>(k_pages);
  a.v_pages = static_cast<uint8_t*>(v_pages);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  // workspace: check words [W][Hkv], partial o [P][Hq][D], partial lse
  // [P][Hq], q' of the prologue [B][Hq][D] bf16, per-request slot ranges
  // [B][2], each from a 256-byte boundary
  uint8_t* ws = static_cast<uint8_t*>(p->workspace);
  const int64_t c_bytes = round256(W * p->n_kv_heads * 4);
  const int64_t o_bytes = round256(P * p->n_q_heads * D * 4);
  const int64_t l_bytes = round256(P * p->n_q_heads * 4);
  const int64_t qp_bytes = round256((int64_t)p->batch * p->n_q_heads * D * 2);
  a.check = ws ? reinterpret_cast<int32_t*>(ws) : nullptr;
  a.part_o = ws ? reinterpret_cast<float*>(ws + c_bytes) : nullptr;
  a.part_lse = ws ? reinterpret_cast<float*>(ws + c_bytes + o_bytes) : nullptr;
  a.q_prime = ws ? reinterpret_cast<uint16_t*>(ws + c_bytes + o_bytes + l_bytes) : nullptr;
  a.req_slots = ws ? reinterpret_cast<int32_t*>(ws + c_bytes + o_bytes + l_bytes + qp_bytes)
                   : nullptr;
  a.cover = nullptr;
  a.q_norm_w = static_cast<const uint16_t*>(p->q_norm_w);
  a.k_norm_w = static_cast<const uint16_t*>(p->k_norm_w);
  a.k_new = static_cast<const uint16_t*>(p->k_new);
  a.v_new = static_cast<const uint16_t*>(p->v_new);
  a.scale_mode = p->scale_mode;
  a.v_dim_major = p->v_layout == HDA_V_DIM_MAJOR;
  a.k_scales = p->scale_mode == HDA_SCALE_TENSOR ? nullptr : p->k_scales;
  a.v_scales = p->scale_mode == HDA_SCALE_TENSOR ? nullptr : p->v_scales;
  a.head_stride = p->page_size * D * elem;
  a.page_stride = (int64_t)a.head_stride * p->n_kv_heads;
  a.num_pages = (int32_t)(p->num_pages < 0x7fffffffLL ? p->num_pages : 0x7fffffffLL);
  a.batch = p->batch;
  a.n_q_heads = p->n_q_heads;
  a.n_kv_heads = p->n_kv_heads;
  a.group = p->n_q_heads / p->n_kv_heads;
  a.page_size = p->page_size;
  a.log2_ps = __builtin_ctz((unsigned)p->page_size);
  a.max_pages = p->max_pages_per_req;
  a.n_wg = (int32_t)W;
  a.n_parts = (int32_t)P;
  a.qb = 1;
  a.n_req = p->batch;
  a.qk_scale_log2 = (float)((double)p->sm_scale * (double)p->k_scale * 1.4426950408889634);
  a.v_scale = p->v_scale;
  a.k_scale = p->k_scale;
  a.rms_eps = p->rms_eps;
  a.rope_theta = p->rope_theta;
  return a;
}

}  // namespace

namespace {

// hda_decode, and with `cover` its coverage-counting debug form (plan in
// device memory only).
int decode_step(const hda_params* p, const void* q, void* k_pages, void* v_pages,
                const int32_t* block_table, const int32_t* seq_lens, const int32_t* plan_host,
                const int32_t* plan_dev, int64_t plan_len, float* out, void* stream,
                int32_t* cover) {
  int st = check_params(p, q, k_pages, v_pages, block_table, seq_lens, out);
  if (st != HDA_OK) return st;
  if (!plan_host) return HDA_ERR_INVALID_ARG;
  if (plan_len < HDA_PLAN_HEADER_INTS || plan_host[0] != HDA_PLAN_VERSION) return HDA_ERR_BAD_PLAN;
  if (!plan_dev && plan_len > kArgPlanInts) return HDA_ERR_UNSUPPORTED;
  if (plan_host[1] != p->batch) return HDA_ERR_PLAN_MISMATCH;
  const int64_t W = plan_host[3], N = plan_host[5], P = plan_host[6];
  if (W < 1 || N < 1 || P < 0 || plan_len != HDA_PLAN_HEADER_INTS + (W + 1) + 4 * N + p->batch + 1)
    return HDA_ERR_BAD_PLAN;
  if (!wg_ranges_ok(plan_host, W, N)) return HDA_ERR_BAD_PLAN;
  const int64_t grid = W * p->n_kv_heads;
  if (grid > 0x7fffffffLL) return HDA_ERR_UNSUPPORTED;
  const int64_t ws_need = hda_workspace_bytes(plan_host, plan_len, p->n_q_heads, p->n_kv_heads,
                                              p->head_dim);
  if (ws_need < 0) return HDA_ERR_BAD_PLAN;
  if ((P > 0 || p->prologue) && (!p->workspace || p->workspace_bytes < ws_need))
    return HDA_ERR_WORKSPACE;

  Args a = make_args(p, q, k_pages, v_pages, block_table, seq_lens, out, W, P);
  // without partial slots or prologue the workspace is optional; the check
  // words are then recorded only when it is large enough
  if (!p->workspace || p->workspace_bytes < ws_need) a.check = nullptr;
  a.plan = plan_dev;
  a.n_items = (int32_t)N;
  a.tile_len = plan_host[2];
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool fp8 = p->kv_dtype == HDA_KV_FP8_E4M3;
  const bool native = p->math == HDA_MATH_FP8;
  const bool pro = p->prologue != 0;
  // the split requests and their slot ranges, for a merge over them alone
  MergeList ml;
  int n_split = 0;
  bool listed = P > 0;
  {
    const int32_t* rpp = plan_host + HDA_PLAN_HEADER_INTS + (W + 1) + 4 * N;
    for (int64_t b = 0; listed && b < p->batch; ++b) {
      const int32_t cnt = rpp[b + 1] - rpp[b];
      if (cnt <= 0) continue;
      if (n_split == kMergeListMax) {
        listed = false;
        break;
      }
      ml.v[3 * n_split] = (int32_t)b;
      ml.v[3 * n_split + 1] = rpp[b];
      ml.v[3 * n_split + 2] = cnt;
      ++n_split;
    }
    if (n_split == 0) listed = false;
  }
  const MergeList* mlp = listed ? &ml : nullptr;
  hipError_t e;
  if (cover) {
    if (!plan_dev) return HDA_ERR_INVALID_ARG;
    a.cover = cover;
    e = p->head_dim == 64 ? launch_d<64, false, true>(a, fp8, native, (int)grid, pro, a.q_prime,
                                                      hs, p->split_event, nullptr, mlp, n_split)
                          : launch_d<128, false, true>(a, fp8, native, (int)grid, pro, a.q_prime,
                                                       hs, p->split_event, nullptr, mlp, n_split);
    return e == hipSuccess ? HDA_OK : HDA_ERR_HIP;
  }
  ArgPlan ap;   // the plan in the launch arguments when no device copy is given
  if (!plan_dev) memcpy(ap.v, plan_host, (size_t)plan_len * sizeof(int32_t));
  const ArgPlan* app = plan_dev ? nullptr : &ap;
  e = p->head_dim == 64 ? launch_d<64, false>(a, fp8, native, (int)grid, pro, a.q_prime, hs,
                                              p->split_event, app, mlp, n_split)
                        : launch_d<128, false>(a, fp8, native, (int)grid, pro, a.q_prime, hs,
                                               p->split_event, app, mlp, n_split);
  return e == hipSuccess ? HDA_OK : HDA_ERR_HIP;
}

}  // namespace

extern "C" int hda_decode(const hda_params* p, const void* q, void* k_pages, void* v_pages,
                          const int32_t* block_table, const int32_t* seq_lens,
                          const int32_t* plan_host, const int32_t* plan_dev, int64_t plan_len,
                          float* out, void* stream) {
  return decode_step(p, q, k_pages, v_pages, block_table, seq_lens, plan_host, plan_dev,
                     plan_len, out, stream, nullptr);
}

// ---- the same step for callers that cannot allocate device memory ----
//
// Its workspace is this array: one copy on every GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory; its device address on the current GPU comes
// from hipGetSymbolAddress, looked up on the first call on each device and
// kept.  Nothing in it needs to start at zero: every region a launch reads
// is written earlier in the same step (check words by each tile workgroup,
// partials by the tile kernel before the merge, q' by the prologue).
namespace {

constexpr int64_t kScratchBytes = HDA_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (stream must run there).
int scratch_address(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HDA_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return HDA_ERR_HIP;
    if (sdev != dev) return HDA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HDA_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return HDA_OK;
}

}  // namespace

extern "C" int hda_decode_noalloc(const hda_params* p, const void* q, void* k_pages,
                                  void* v_pages, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* plan_host,
                                  const int32_t* plan_dev, int64_t plan_len, float* out,
                                  void* stream) {
  if (!p) return HDA_ERR_INVALID_ARG;
  void* ws = nullptr;
  const int st = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (st != HDA_OK) return st;
  hda_params local = *p;
  local.workspace = ws;
  local.workspace_bytes = kScratchBytes;   // a larger plan: HDA_ERR_WORKSPACE
  return decode_step(&local, q, k_pages, v_pages, block_table, seq_lens, plan_host, plan_dev,
                     plan_len, out, stream, nullptr);
}

extern "C" int hda_decode_coverage(const hda_params* p, const void* q, void* k_pages,
                                   void* v_pages, const int32_t* block_table,
                                   const int32_t* seq_lens, const int32_t* plan_host,
                                   const int32_t* plan_dev, int64_t plan_len, float* out,
                                   int32_t* visits, void* stream) {
  if (!visits || !plan_dev) return HDA_ERR_INVALID_ARG;
  return decode_step(p, q, k_pages, v_pages, block_table, seq_lens, plan_host, plan_dev,
                     plan_len, out, stream, visits);
}

extern "C" int hda_decode_check(const hda_params* p, int32_t n_workgroups, int32_t* flags,
                                void* stream) {
  if (!p || !flags || n_workgroups < 1 || p->n_kv_heads < 1 || !p->workspace)
    return HDA_ERR_INVALID_ARG;
  const int64_t n = (int64_t)n_workgroups * p->n_kv_heads;
  if (p->workspace_bytes < n * 4) return HDA_ERR_INVALID_ARG;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t buf[1024];
  int32_t bits = 0;
  for (int64_t off = 0; off < n; off += 1024) {
    const int64_t m = n - off < 1024 ? n - off : 1024;
    if (hipMemcpyAsync(buf, static_cast<const int32_t*>(p->workspace) + off, (size_t)m * 4,
                       hipMemcpyDeviceToHost, hs) != hipSuccess ||
        hipStreamSynchronize(hs) != hipSuccess)
      return HDA_ERR_HIP;
    for (int64_t i = 0; i < m; ++i) bits |= buf[i];
  }
  *flags = bits;
  return bits ? HDA_ERR_PLAN_MISMATCH : HDA_OK;
}

extern "C" int64_t hda_workspace_bytes_bound(int32_t batch, int32_t n_workgroups,
                                             int32_t n_q_heads, int32_t head_dim) {
  if (batch < 1 || n_workgroups < 1 || n_q_heads < 1 || head_dim < 1) return -1;
  const int64_t P = (int64_t)n_workgroups + batch - 1;   // partial slots <= items <= W + B - 1
  // check words counted as W x Hq (>= W x Hkv, the count a launch writes)
  return round256((int64_t)n_workgroups * n_q_heads * 4) + round256(P * n_q_heads * head_dim * 4) +
         round256(P * n_q_heads * 4) + round256((int64_t)batch * n_q_heads * head_dim * 2) +
         round256((int64_t)batch * 8);
}

extern "C" int hda_decode_auto(const hda_params* p, const void* q, void* k_pages, void* v_pages,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int32_t tile_len, int32_t n_workgroups, float* out, void* stream) {
  int st = check_params(p, q, k_pages, v_pages, block_table, seq_lens, out);
  if (st != HDA_OK) return st;
  if (tile_len < 1 || n_workgroups < 1) return HDA_ERR_INVALID_ARG;
  if ((int64_t)n_workgroups + p->batch > 0x7fffffffLL) return HDA_ERR_INVALID_ARG;
  const int64_t grid = (int64_t)n_workgroups * p->n_kv_heads;
  if (grid > 0x7fffffffLL) return HDA_ERR_UNSUPPORTED;
  const int64_t ws_need = hda_workspace_bytes_bound(p->batch, n_workgroups, p->n_q_heads,
                                                    p->head_dim);
  if (!p->workspace || p->workspace_bytes < ws_need) return HDA_ERR_WORKSPACE;
  const int64_t P = (int64_t)n_workgroups + p->batch - 1;
  Args a = make_args(p, q, k_pages, v_pages, block_table, seq_lens, out, n_workgroups, P);
  a.plan = nullptr;
  a.n_items = 0;
  a.tile_len = tile_len;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool fp8 = p->kv_dtype == HDA_KV_FP8_E4M3;
  const bool native = p->math == HDA_MATH_FP8;
  const bool pro = p->prologue != 0;
  hipError_t e =
      p->head_dim == 64
          ? launch_d<64, true>(a, fp8, native, (int)grid, pro, a.q_prime, hs, p->split_event)
          : launch_d<128, true>(a, fp8, native, (int)grid, pro, a.q_prime, hs, p->split_event);
  return e == hipSuccess ? HDA_OK : HDA_ERR_HIP;
}

extern "C" int hda_prefill(const hda_params* p, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* block_table,
                           const int32_t* kv_lens, int32_t n_q, const int32_t* rows_host,
                           const int32_t* rows_dev, const int32_t* plan_host,
                           const int32_t* plan_dev, int64_t plan_len, float* out, void* stream) {
  int st = check_params(p, q, k_pages, v_pages, block_table, kv_lens, out);
  if (st != HDA_OK) return st;
  if (p->prologue || p->math != HDA_MATH_BF16 || p->v_layout != HDA_V_TOKEN_MAJOR)
    return HDA_ERR_UNSUPPORTED;
  if (!rows_host || !rows_dev || !plan_host || !plan_dev || n_q < 1) return HDA_ERR_INVALID_ARG;
  if (plan_len < HDA_PLAN_HEADER_INTS || plan_host[0] != HDA_PLAN_VERSION) return HDA_ERR_BAD_PLAN;
  const int64_t R = plan_host[1], W = plan_host[3], N = plan_host[5], P = plan_host[6];
  if (R < 1 || W < 1 || N < 1 || P < 0 || plan_len != HDA_PLAN_HEADER_INTS + (W + 1) + 4 * N + R + 1)
    return HDA_ERR_BAD_PLAN;
  if (!wg_ranges_ok(plan_host, W, N)) return HDA_ERR_BAD_PLAN;
  const int32_t unit = hda_prefill_rows_per_block(p->n_q_heads, p->n_kv_heads);
  if (unit < 1) return HDA_ERR_UNSUPPORTED;
  // every block inside its request and the packed q (the kernel trusts
  // them); the largest block sets the partial-slot stride and the kernel
  int32_t qb = 1;
  for (int64_t r = 0; r < R; ++r) {
    const int32_t b = rows_host[4 * r], q0 = rows_host[4 * r + 1], nq = rows_host[4 * r + 2],
                  pos0 = rows_host[4 * r + 3];
    if (b < 0 || b >= p->batch || nq < 1 || nq > HDA_PREFILL_MAX_TILES * unit || q0 < 0 ||
        (int64_t)q0 + nq > n_q || pos0 < 0)
      return HDA_ERR_INVALID_ARG;
    qb = nq > qb ? nq : qb;
  }
  const int64_t grid = W * p->n_kv_heads;
  if (grid > 0x7fffffffLL || R * qb * p->n_q_heads > 0x7fffffffLL) return HDA_ERR_UNSUPPORTED;
  const int64_t ws_need = hda_prefill_workspace_bytes(plan_host, plan_len, p->n_q_heads,
                                                      p->n_kv_heads, p->head_dim, qb);
  if (ws_need < 0) return HDA_ERR_BAD_PLAN;
  if (P > 0 && (!p->workspace || p->workspace_bytes < ws_need)) return HDA_ERR_WORKSPACE;
  // without partial slots a smaller workspace may still hold the check words
  const bool ws_ok = p->workspace && p->workspace_bytes >= ws_need;

  Args a = make_args(p, q, const_cast<void*>(k_pages), const_cast<void*>(v_pages), block_table,
                     kv_lens, out, W, 0);
  // workspace: check words [W][Hkv], partial o [P][qb][Hq][D], partial lse
  // [P][qb][Hq], each from a 256-byte boundary
  uint8_t* ws = ws_ok ? static_cast<uint8_t*>(p->workspace) : nullptr;
  const int64_t c_bytes = round256(W * p->n_kv_heads * 4);
  const int64_t o_bytes = round256((int64_t)P * qb * p->n_q_heads * p->head_dim * 4);
  a.check = ws ? reinterpret_cast<int32_t*>(ws) : nullptr;
  a.part_o = ws ? reinterpret_cast<float*>(ws + c_bytes) : nullptr;
  a.part_lse = ws ? reinterpret_cast<float*>(ws + c_bytes + o_bytes) : nullptr;
  a.q_prime = nullptr;
  a.req_slots = nullptr;
  a.n_parts = (int32_t)P;
  a.qb = qb;
  a.batch = (int32_t)R;              // the plan's requests are the row blocks
  a.rows = rows_dev;
  a.plan = plan_dev;
  a.n_items = (int32_t)N;
  a.tile_len = plan_host[2];
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool fp8 = p->kv_dtype == HDA_KV_FP8_E4M3;
  // the largest slot count of a block (the merge's early loads)
  int max_slots = 0;
  {
    const int32_t* rpp = plan_host + HDA_PLAN_HEADER_INTS + (W + 1) + 4 * N;
    for (int64_t r = 0; r < R; ++r) max_slots = std::max(max_slots, rpp[r + 1] - rpp[r]);
  }
  hipError_t e = p->head_dim == 64
                     ? launch_prefill_d<64>(a, fp8, (int)grid, (int)R, max_slots, hs,
                                            p->split_event)
                     : launch_prefill_d<128>(a, fp8, (int)grid, (int)R, max_slots, hs,
                                             p->split_event);
  return e == hipSuccess ? HDA_OK : HDA_ERR_HIP;
}

extern "C" int hda_plan_upload(const int32_t* plan_host, int64_t plan_len, int32_t* plan_dev,
                               void* stream) {
  if (!plan_host || !plan_dev || plan_len < 1 || ((uintptr_t)plan_dev & 3u))
    return HDA_ERR_INVALID_ARG;
  UploadChunk c;
  for (int64_t off = 0; off < plan_len; off += kUploadInts) {
    const int n = (int)(plan_len - off < kUploadInts ? plan_len - off : kUploadInts);
    memcpy(c.v, plan_host + off, (size_t)n * sizeof(int32_t));
    hipLaunchKernelGGL(hda_plan_store_kernel, dim3(1), dim3(256), 0,
                       static_cast<hipStream_t>(stream), c, plan_dev + off, n);
    if (hipGetLastError() != hipSuccess) return HDA_ERR_HIP;
  }
  return HDA_OK;
}

extern "C" int hda_plan_device(const int32_t* seq_lens, int32_t batch, int32_t tile_len,
                               int32_t n_workgroups, int32_t* plan, int64_t capacity,
                               void* stream) {
  if (!seq_lens || !plan || batch < 1 || tile_len < 1 || n_workgroups < 1)
    return HDA_ERR_INVALID_ARG;
  if ((int64_t)n_workgroups + batch > 0x7fffffffLL) return HDA_ERR_INVALID_ARG;
  if (capacity < hda_plan_capacity(batch, n_workgroups)) return HDA_ERR_CAPACITY;
  hipLaunchKernelGGL(hda_plan_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     seq_lens, batch, tile_len, n_workgroups, plan);
  return hipGetLastError() == hipSuccess ? HDA_OK : HDA_ERR_HIP;
}

// Router GEMM for MI355X (gfx950): MoE routing logits from bf16 activations
// and fp32 weights kept as two bf16 parts.
//
// The pages describe the operator: fp32 router weights become a bf16 high
// part and a bf16 residual stored with a scale of 1/256; two bf16 matrix
// products run in one kernel, sharing the input movement and keeping their
// accumulators in registers, and are combined once ("Tencent HPC llega a
// SGLang ...", remio.ai, Router GEMM section; arex-research page, Router
// GEMM paragraph).  Here: hi = bf16(w), lo = bf16(256 (w - hi)), and
//   out[t][e] = sum_h x[t][h] hi[e][h] + (sum_h x[t][h] lo[e][h]) / 256
// with fp32 accumulation on v_mfma_f32_16x16x32_bf16.
//
// Tiling (65 to a few hundred tokens; 9 to 64 take the one-launch split
// kernel further down, fewer the one-workgroup-per-expert kernel, more the
// LDS-staged kernel).  A workgroup owns TM tokens (32 or 64) x 64 experts
// and a range of the hidden dimension; its 4 waves take interleaved 32-wide K steps of that
// range, each holding the full TM x 64 tile for both products (2 x TM/16 x 4
// MFMA blocks), and combine through LDS at the end.  The activation fragment
// of a K step is loaded once and feeds both products.  When the token and
// expert tiles alone give too few workgroups for 256 compute units (decode
// batches), the hidden dimension is also split S ways across workgroups;
// their partial tiles go to the workspace and a second kernel adds them in a
// fixed order (deterministic).  Rows past T or E read as zero through the
// buffer range checks.
#include <hip/hip_runtime.h>
#include <stdint.h>


#include "hda.h"
#include "hda_arrive.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kRsrcWord3 = 0x00020000;
constexpr int kWaves = 4;
constexpr int kTileE = 64;        // experts per workgroup tile
constexpr int kStepK = 32;        // K per MFMA
constexpr float kResidualScale = 1.0f / 256.0f;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffffLL ? 0x7fffffff : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

__device__ inline bf16x8 load8(const __amdgpu_buffer_rsrc_t& r, int64_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

struct RouterArgs {
  const uint16_t* x;     // bf16 [T][H]
  const uint16_t* w_hi;  // bf16 [E][H]
  const uint16_t* w_lo;  // bf16 [E][H], residual x 256
  float* out;            // fp32 [T][E]
  float* part;           // fp32 [S][T][E] when S > 1
  int32_t T, E, H;
  int32_t k_per_wg;      // hidden range per workgroup (multiple of 4 x 32)
};

// TM = 16 * MB tokens per tile.  Lane (i, kg) of a 16x16x32 MFMA block holds
// row i, k = 8 kg .. 8 kg + 7 of both operands; the C layout is
// C[4 kg + r][i].
template <int MB>
__global__ __launch_bounds__(64 * kWaves) void hda_router_gemm_kernel(RouterArgs a) {
  constexpr int TM = 16 * MB;
  __shared__ float red[kWaves][TM][kTileE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, kg = lane >> 4;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * kTileE, s = blockIdx.z;
  const int kb = s * a.k_per_wg;
  const int ke = min(a.H, kb + a.k_per_wg);

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (int64_t)a.T * a.H * 2);
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.w_hi, (int64_t)a.E * a.H * 2);
  const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.w_lo, (int64_t)a.E * a.H * 2);

  f32x4 acc_hi[MB][4], acc_lo[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      acc_hi[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_lo[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // byte offsets of this lane's rows at k = 0
  int64_t xoff[MB], woff[4];
#pragma unroll
  for (int m = 0; m < MB; ++m) xoff[m] = ((int64_t)(t0 + 16 * m + i) * a.H + 8 * kg) * 2;
#pragma unroll
  for (int n = 0; n < 4; ++n) woff[n] = ((int64_t)(e0 + 16 * n + i) * a.H + 8 * kg) * 2;

  // two fragment sets: the loads of the wave's next K step are in flight
  // while the current step multiplies
  struct Frags {
    bf16x8 xa[MB], wh[4], wl[4];
  };
  auto load = [&](Frags& f, int k) {
#pragma unroll
    for (int m = 0; m < MB; ++m) f.xa[m] = load8(xr, xoff[m] + 2 * k);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      f.wh[n] = load8(hr, woff[n] + 2 * k);
      f.wl[n] = load8(lr, woff[n] + 2 * k);
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        acc_hi[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.xa[m], f.wh[n], acc_hi[m][n], 0, 0, 0);
        acc_lo[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.xa[m], f.wl[n], acc_lo[m][n], 0, 0, 0);
      }
  };
  constexpr int kStride = kStepK * kWaves;
  Frags f0, f1;
  int k = kb + kStepK * wave;
  if (k < ke) load(f0, k);
  while (k < ke) {
    const int k1 = k + kStride;
    if (k1 < ke) load(f1, k1);
    mma(f0);
    if (k1 >= ke) break;
    const int k2 = k1 + kStride;
    if (k2 < ke) load(f0, k2);
    mma(f1);
    k = k2;
  }
  // combine the two products, then the four waves
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[wave][16 * m + 4 * kg + r][16 * n + i] = acc_hi[m][n][r] + acc_lo[m][n][r] * kResidualScale;
  __syncthreads();
  float* dst = gridDim.z > 1 ? a.part + (int64_t)s * a.T * a.E : a.out;
  for (int idx = tid; idx < TM * kTileE; idx += 64 * kWaves) {
    const int tt = idx / kTileE, ee = idx - tt * kTileE;
    const int t = t0 + tt, e = e0 + ee;
    if (t < a.T && e < a.E)
      dst[(int64_t)t * a.E + e] = (red[0][tt][ee] + red[1][tt][ee]) + (red[2][tt][ee] + red[3][tt][ee]);
  }
}

// Large batches: 128 tokens x 128 experts per workgroup, K sliced by 64 (two
// MFMA steps per barrier; slices of 32 measured 10% slower) and staged
// through LDS (two stages) from registers loaded two slices ahead (two
// register sets; one slice ahead left each step waiting ~3x its MFMA time
// on memory).  Eight waves: wave (wm, wn) owns the 64 x 32 sub-tile at
// (64 wm, 32 wn), 4 x 2 blocks for each product, which keeps the
// accumulators and both register sets within 256 registers (two waves per
// SIMD).  LDS tiles are swizzled (big_off) so that fragment reads are
// conflict-free.
constexpr int kBigM = 128, kBigN = 128;
constexpr int kBigK = 64;             // K per LDS stage (two MFMA steps)

// A tile of 128 rows of 64 bf16 (8 16-byte quads): rows r and r + 8 of each
// 16 share a 256-byte line, quad q of row r in half (q / 4) ^ (r / 8 mod 2)
// at position (r ^ q) mod 8, so that the 16 rows of a fragment read (one
// quad each) put lanes 0-7 and lanes 8-15 each on one aligned half of the
// banks (the rule gfx950's 16-byte reads are conflict-free under).
struct BigStage {
  uint8_t a[kBigM * 2 * kBigK];
  uint8_t bh[kBigN * 2 * kBigK];
  uint8_t bl[kBigN * 2 * kBigK];
};
__device__ inline int big_off(int r, int q) {
  return (r >> 4) * 2048 + (r & 7) * 256 + 16 * (8 * ((q >> 2) ^ ((r >> 3) & 1)) + ((r ^ q) & 7));
}

constexpr int kBigWaves = 8;          // 2 x 4 waves of 64 x 32 sub-tiles

__global__ __launch_bounds__(64 * kBigWaves, 1) void hda_router_gemm_lds_kernel(RouterArgs a) {
  __shared__ BigStage st[2];
  constexpr int NT = 64 * kBigWaves;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, kg = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;         // rows 64 wm.., experts 32 wn..
  const int t0 = blockIdx.x * kBigM, e0 = blockIdx.y * kBigN;
  const int kb = blockIdx.z * a.k_per_wg;
  const int ke = min(a.H, kb + a.k_per_wg);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (int64_t)a.T * a.H * 2);
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.w_hi, (int64_t)a.E * a.H * 2);
  const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.w_lo, (int64_t)a.E * a.H * 2);

  // global -> LDS copy: 1024 16-byte chunks per tile, two per thread; chunk
  // c is row c / 8, k offset 8 (c % 8)
  constexpr int kChunks = kBigM * kBigK / 8 / NT;    // per thread per tile
  int64_t ga[kChunks], gb[kChunks];
  int lrow[kChunks], lcol[kChunks];
#pragma unroll
  for (int u = 0; u < kChunks; ++u) {
    const int c = tid + NT * u;
    lrow[u] = c >> 3;
    lcol[u] = 8 * (c & 7);
    ga[u] = ((int64_t)(t0 + lrow[u]) * a.H + lcol[u]) * 2;
    gb[u] = ((int64_t)(e0 + lrow[u]) * a.H + lcol[u]) * 2;
  }
  // two register sets: the slice two steps ahead is in flight while the
  // next one waits to be stored
  struct Regs { u32x4 a[kChunks], h[kChunks], l[kChunks]; } r0, r1;
  auto load = [&](Regs& r, int k) {
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      // (the K offset as the scalar offset: no per-step address arithmetic
      // in registers the compiler might then have to wait for)
      r.a[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)ga[u], 2 * k, 0));
      r.h[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hr, (int)gb[u], 2 * k, 0));
      r.l[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(lr, (int)gb[u], 2 * k, 0));
    }
  };
  auto store = [&](const Regs& r, BigStage& s) {
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int off = big_off(lrow[u], lcol[u] / 8);
      *reinterpret_cast<u32x4*>(s.a + off) = r.a[u];
      *reinterpret_cast<u32x4*>(s.bh + off) = r.h[u];
      *reinterpret_cast<u32x4*>(s.bl + off) = r.l[u];
    }
  };

  f32x4 acc_hi[4][2], acc_lo[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      acc_hi[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_lo[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  auto compute = [&](const BigStage& s) {
#pragma unroll
    for (int kk = 0; kk < kBigK; kk += kStepK) {
      bf16x8 fa[4], fh[2], fl[2];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        fa[m] = *reinterpret_cast<const bf16x8*>(s.a + big_off(64 * wm + 16 * m + i, kk / 8 + kg));
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        fh[n] = *reinterpret_cast<const bf16x8*>(s.bh + big_off(32 * wn + 16 * n + i, kk / 8 + kg));
        fl[n] = *reinterpret_cast<const bf16x8*>(s.bl + big_off(32 * wn + 16 * n + i, kk / 8 + kg));
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          acc_hi[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[m], fh[n], acc_hi[m][n], 0, 0, 0);
          acc_lo[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[m], fl[n], acc_lo[m][n], 0, 0, 0);
        }
    }
  };
  // slices alternate between LDS stages 0 and 1 and register sets r0 and
  // r1 (the loop is unrolled by two so that both are named statically)
  const int nk = (ke - kb) / kBigK;
  load(r0, kb);
  store(r0, st[0]);
  __syncthreads();
  if (nk > 1) load(r1, kb + kBigK);
  // The loads two slices ahead are always issued (the last slice again
  // past the end; nothing stores those): with a branch around them the
  // wait before storing the next slice would count the loads of both paths
  // and drain the ones in flight.
  for (int ks = 0; ks < nk; ks += 2) {
    load(r0, kb + kBigK * min(ks + 2, nk - 1));
    compute(st[0]);
    if (ks + 1 < nk) store(r1, st[1]);
    __syncthreads();
    if (ks + 1 >= nk) break;
    load(r1, kb + kBigK * min(ks + 3, nk - 1));
    compute(st[1]);
    if (ks + 2 < nk) store(r0, st[0]);
    __syncthreads();
  }
  float* dst = gridDim.z > 1 ? a.part + (int64_t)blockIdx.z * a.T * a.E : a.out;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 64 * wm + 16 * m + 4 * kg + r, e = e0 + 32 * wn + 16 * n + i;
        if (t < a.T && e < a.E)
          dst[(int64_t)t * a.E + e] = acc_hi[m][n][r] + acc_lo[m][n][r] * kResidualScale;
      }
}

// Small token counts (T <= 8): one launch, no hidden split and no second
// kernel.  Workgroup b computes out[t][EPW b + j] for every token t < T and
// its EPW experts over the whole hidden dimension: thread tid takes the
// 8-element vectors tid, tid + 256, ..., loading each vector of x (every
// token) and of both weight parts once, all of a batch's loads issued
// before its arithmetic; both products accumulate in float32 per thread,
// then a butterfly within each wave and the four waves in order
// (deterministic).  Matrix cores would need 16-expert tiles, i.e. 16
// workgroups streaming 0.46 MB each at hidden 7168; here the weights spread
// over E / EPW workgroups (256 at EPW 1: 28 KB each) and x comes from L2.
// Rows past T or E and vectors past H read as zero through the buffer range
// checks.
constexpr int kGemvThreadsDefault = 256;

__device__ inline void bf16x8_to_f32(const bf16x8& v, float (&f)[8]) {
  const u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(u[q] << 16);
    f[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
  }
}

template <int TT, int EPW, int kGemvThreads = kGemvThreadsDefault>
__global__ __launch_bounds__(kGemvThreads) void hda_router_gemv_kernel(RouterArgs a) {
  constexpr int kGemvBatch = 1024 / kGemvThreads;   // vectors per thread in flight
  constexpr int kWv = kGemvThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = blockIdx.x * EPW;
  const int nv = a.H / 8;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (int64_t)a.T * a.H * 2);
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.w_hi, (int64_t)a.E * a.H * 2);
  const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.w_lo, (int64_t)a.E * a.H * 2);
  constexpr int kOut = 0x7ffffff0;     // an offset past every range: reads zero
  float ah[TT][EPW], al[TT][EPW];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int j = 0; j < EPW; ++j) ah[t][j] = al[t][j] = 0.f;
  for (int v0 = 0; v0 < nv; v0 += kGemvThreads * kGemvBatch) {
    bf16x8 xv[kGemvBatch][TT], hv[kGemvBatch][EPW], lv[kGemvBatch][EPW];
#pragma unroll
    for (int u = 0; u < kGemvBatch; ++u) {
      const int v = v0 + tid + kGemvThreads * u;
      const bool in = v < nv;
#pragma unroll
      for (int t = 0; t < TT; ++t)
        xv[u][t] = load8(xr, in ? ((int64_t)t * a.H + 8 * v) * 2 : kOut);
#pragma unroll
      for (int j = 0; j < EPW; ++j) {
        const int64_t off = in ? ((int64_t)(e0 + j) * a.H + 8 * v) * 2 : kOut;
        hv[u][j] = load8(hr, off);
        lv[u][j] = load8(lr, off);
      }
    }
#pragma unroll
    for (int u = 0; u < kGemvBatch; ++u) {
      float wh[EPW][8], wl[EPW][8];
#pragma unroll
      for (int j = 0; j < EPW; ++j) {
        bf16x8_to_f32(hv[u][j], wh[j]);
        bf16x8_to_f32(lv[u][j], wl[j]);
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        float xf[8];
        bf16x8_to_f32(xv[u][t], xf);
#pragma unroll
        for (int j = 0; j < EPW; ++j)
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            ah[t][j] = __builtin_fmaf(xf[k], wh[j][k], ah[t][j]);
            al[t][j] = __builtin_fmaf(xf[k], wl[j][k], al[t][j]);
          }
      }
    }
  }
  __shared__ float red[kWv][TT * EPW][2];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
      float h = ah[t][j], l = al[t][j];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        h += __shfl_xor(h, o);
        l += __shfl_xor(l, o);
      }
      if (lane == 0) {
        red[wave][t * EPW + j][0] = h;
        red[wave][t * EPW + j][1] = l;
      }
    }
  __syncthreads();
  if (tid < TT * EPW) {
    const int t = tid / EPW, e = e0 + tid % EPW;
    float h = red[0][tid][0], l = red[0][tid][1];
#pragma unroll
    for (int ww = 1; ww < kWv; ++ww) {
      h += red[ww][tid][0];
      l += red[ww][tid][1];
    }
    if (t < a.T && e < a.E) a.out[(int64_t)t * a.E + e] = h + l * kResidualScale;
  }
}

// Decode-sized batches (9 to 64 tokens) in one launch.  A workgroup owns
// TM = 16 MB tokens x 16 experts (one MFMA block wide) and a range of the
// hidden dimension: with 16-expert tiles, 16 ranges give 256 workgroups at
// 256 experts, each streaming 28 KB of weights.  Its 4 waves take
// interleaved 32-wide K steps of the range, every load of a group of NS
// steps issued before the group's first MFMA (steps past the range read
// zeros through the range checks), and combine through LDS.  With S > 1
// ranges the workgroup stores its partial tile in the workspace and arrives
// at the tile's counter; the last of the S workgroups to arrive adds the S
// partials in slot order and writes the logits, so the result does not
// depend on which workgroup came last.
//
// Counter words of the output tiles: the last-arriver protocol of
// hda_arrive.h with this kernel's signature.
constexpr uint32_t kCounterSig = 0x52544731u;

constexpr int kFusedTN = 16;          // experts per fused tile
constexpr int kFusedNS = 4;           // K steps per wave per load group

template <int MB>
__global__ __launch_bounds__(64 * kWaves) void hda_router_fused_kernel(RouterArgs a, float* part,
                                                                      unsigned long long* cnt) {
  constexpr int TM = 16 * MB, TN = kFusedTN, NT = TM * TN, NS = kFusedNS;
  __shared__ float red[kWaves][NT];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, kg = lane >> 4;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TN, s = blockIdx.z, S = gridDim.z;
  const int kb = s * a.k_per_wg;
  const int ke = min(a.H, kb + a.k_per_wg);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (int64_t)a.T * a.H * 2);
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.w_hi, (int64_t)a.E * a.H * 2);
  const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.w_lo, (int64_t)a.E * a.H * 2);
  constexpr int kOut = 0x7ffffff0;     // an offset past every range: reads zero

  f32x4 acc_hi[MB], acc_lo[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc_hi[m] = acc_lo[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  int64_t xoff[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) xoff[m] = ((int64_t)(t0 + 16 * m + i) * a.H + 8 * kg) * 2;
  const int64_t woff = ((int64_t)(e0 + i) * a.H + 8 * kg) * 2;
  for (int g = kb + kStepK * wave; g < ke; g += kStepK * kWaves * NS) {
    bf16x8 xa[NS][MB], wh[NS], wl[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int k = g + kStepK * kWaves * j;
      const bool in = k < ke;
#pragma unroll
      for (int m = 0; m < MB; ++m) xa[j][m] = load8(xr, in ? xoff[m] + 2 * k : kOut);
      wh[j] = load8(hr, in ? woff + 2 * k : kOut);
      wl[j] = load8(lr, in ? woff + 2 * k : kOut);
    }
    // keep the scheduler from interleaving the loads with the products
    // (it would reuse a few registers and serialise the round trips)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        acc_hi[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j][m], wh[j], acc_hi[m], 0, 0, 0);
        acc_lo[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j][m], wl[j], acc_lo[m], 0, 0, 0);
      }
  }
  // combine the two products, then the four waves; element (tt, ee) of the
  // tile at tt * TN + ee
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      red[wave][(16 * m + 4 * kg + r) * TN + i] = acc_hi[m][r] + acc_lo[m][r] * kResidualScale;
  __syncthreads();
  // thread q < NT / 4 owns elements 4q .. 4q + 3: token 4q / TN, four experts
  const int q = tid;
  const bool owner = q < NT / 4;
  const int tt = 4 * q / TN, ee = 4 * q % TN;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (owner) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = 4 * q + c;
      v[c] = (red[0][idx] + red[1][idx]) + (red[2][idx] + red[3][idx]);
    }
  }
  const int tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (S > 1) {
    if (owner) reinterpret_cast<f32x4*>(part + ((int64_t)tile * S + s) * NT)[q] = v;
    // Every wave waits for its own stores to reach the L2; after the barrier
    // one wave releases the partial tile (an L2 write-back) and arrives.  A
    // release in every wave, or a full fence (which also invalidates the
    // L2), multiplied that cost.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (wave == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if (lane == 0) s_last = hda_arrive_last<kCounterSig>(cnt + tile, S);
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the other workgroups' partials
    if (owner) {
      // every load of a batch issued (indices clamped, no branches) before
      // the first addition; the additions keep slot order
      constexpr int kB = 16;           // partials in flight per thread
      const f32x4* src = reinterpret_cast<const f32x4*>(part + (int64_t)tile * S * NT) + q;
      for (int s0 = 0; s0 < S; s0 += kB) {
        f32x4 pv[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) pv[u] = src[(int64_t)min(s0 + u, S - 1) * (NT / 4)];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kB; ++u)
          if (s0 + u < S) v = (s0 + u == 0) ? pv[u] : v + pv[u];
      }
    }
    if (tid == 0) hda_counter_rest<kCounterSig>(cnt + tile);
  }
  const int t = t0 + tt;
  if (owner && t < a.T) {
    float* o = a.out + (int64_t)t * a.E + e0 + ee;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (e0 + ee + c < a.E) o[c] = v[c];
  }
}

// Sum of the S partial tiles, in slot order.  The loads of a batch of
// kBatch partials are all issued before any is added (one memory round trip
// per batch instead of one per partial); the additions keep slot order.
// Batches of 64 for many splits (small token counts: 56 splits at hidden
// 7168 take one round trip instead of four), of 16 for few (a 64-wide batch
// of mostly idle loads slowed the million-output reductions of large token
// counts by a quarter).
template <int kBatch>
__global__ __launch_bounds__(256) void hda_router_reduce_kernel(const float* __restrict__ part,
                                                                float* __restrict__ out,
                                                                int64_t n, int S) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  float acc = 0.f;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = s0 + u < S ? part[(int64_t)(s0 + u) * n + j] : 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (s0 + u < S) acc = (s0 + u == 0) ? v[u] : acc + v[u];
  }
  out[j] = acc;
}

// w -> (hi, lo): hi = bf16(w), lo = bf16(256 (w - hi)), both rounded to
// nearest even (w - hi is exact in float32, and so is the scaling).
__global__ __launch_bounds__(256) void hda_router_split_kernel(const float* __restrict__ w,
                                                               uint16_t* __restrict__ hi,
                                                               uint16_t* __restrict__ lo,
                                                               int64_t n) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const float v = w[j];
  const __bf16 h = (__bf16)v;
  hi[j] = __builtin_bit_cast(uint16_t, h);
  lo[j] = __builtin_bit_cast(uint16_t, (__bf16)((v - (float)h) * 256.0f));
}

// Launch shape: token tile, expert tiles, and the hidden split S.
struct RouterShape {
  int mb, tiles_t, tiles_e, S, k_per_wg;
  bool big;    // the LDS-staged 128 x 128 kernel
  bool fused;  // the one-launch split kernel (16-expert tiles, last arriver adds)
  int gemv;    // > 0: the one-launch small-batch kernel for up to this many tokens
};

// Token counts up to this take the one-launch kernel (no hidden split).
constexpr int kGemvMaxT = 8;
// Token counts up to this take the one-launch split kernel.
constexpr int kFusedMaxT = 64;
// Its hidden split: tiles x ranges about one workgroup per compute unit.
constexpr int64_t kFusedTargetGroups = 256;

// The LDS-staged 128 x 128 kernel takes a batch when its tiles, split along
// the hidden dimension into ranges of at least 4 LDS stages (256 of K),
// reach 256 workgroups (one per compute unit); smaller batches take the
// split-K register kernel (measured: 64 large tiles alone leave three
// quarters of the compute units idle; ranges of at least 8 stages kept 1024
// tokens on the register kernel, 27.6 us against 20.8).
constexpr int64_t kBigMinGroups = 256;
constexpr int kBigMinStages = 4;      // K per workgroup >= 4 stages (256)
// The split-K register kernel splits the hidden dimension until its tiles
// make about this many workgroups (one per compute unit: measured against
// 128, 192, 384 and 512 over 1 to 16384 tokens, best at 256 and 1024 tokens
// -- fewer partial tiles to write and add -- and equal elsewhere).
constexpr int64_t kSmallTargetGroups = 256;

RouterShape router_shape(int32_t T, int32_t E, int32_t H) {
  RouterShape r{};
  if (T <= kGemvMaxT) {
    r.gemv = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
    r.S = 1;
    return r;
  }
  if (T <= kFusedMaxT) {
    r.fused = true;
    r.mb = T <= 16 ? 1 : T <= 32 ? 2 : 4;
    r.tiles_t = 1;
    r.tiles_e = (E + kFusedTN - 1) / kFusedTN;
    const int steps_total = H / kStepK;                    // H is a multiple of 32
    int64_t S = (kFusedTargetGroups + r.tiles_e - 1) / r.tiles_e;
    S = S < 1 ? 1 : (S > steps_total ? steps_total : S);
    r.k_per_wg = (int)((steps_total + S - 1) / S) * kStepK;
    r.S = (H + r.k_per_wg - 1) / r.k_per_wg;
    return r;
  }
  const int64_t big_tiles = (int64_t)((T + kBigM - 1) / kBigM) * ((E + kBigN - 1) / kBigN);
  const int64_t max_split = H % kBigK ? 0 : H / (kBigK * kBigMinStages);
  if (max_split >= 1 && big_tiles * max_split >= kBigMinGroups) {
    r.big = true;
    r.mb = 8;
    r.tiles_t = (T + kBigM - 1) / kBigM;
    r.tiles_e = (E + kBigN - 1) / kBigN;
    int64_t S = (kBigMinGroups + big_tiles - 1) / big_tiles;
    S = S < 1 ? 1 : (S > max_split ? max_split : S);
    const int stages = H / kBigK;
    r.k_per_wg = (int)((stages + S - 1) / S) * kBigK;
    r.S = (H + r.k_per_wg - 1) / r.k_per_wg;
    return r;
  }
  r.big = false;
  r.mb = T <= 32 ? 2 : 4;
  r.tiles_t = (T + 16 * r.mb - 1) / (16 * r.mb);
  r.tiles_e = (E + kTileE - 1) / kTileE;
  const int64_t base = (int64_t)r.tiles_t * r.tiles_e;
  constexpr int kRound = kStepK * kWaves;                 // one K step per wave
  const int rounds_total = (H + kRound - 1) / kRound;     // >= 1 for H >= 1; last may be partial
  int64_t S = (kSmallTargetGroups + base - 1) / base;
  S = S < 1 ? 1 : (S > rounds_total ? rounds_total : S);
  const int rounds = (int)((rounds_total + S - 1) / S);   // per workgroup, >= 1
  r.k_per_wg = rounds * kRound;
  r.S = (H + r.k_per_wg - 1) / r.k_per_wg;
  return r;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Fused kernel's workspace: one 8-byte counter per tile (rounded up to 256
// bytes), then S partial tiles of 16 MB x 16 floats per tile.
int64_t fused_counter_bytes(const RouterShape& r) {
  return ((int64_t)r.tiles_t * r.tiles_e * 8 + 255) / 256 * 256;
}

int64_t ws_bytes(const RouterShape& r, int32_t tokens, int32_t experts) {
  if (r.S <= 1) return 0;
  if (r.fused)
    return fused_counter_bytes(r) +
           (int64_t)r.tiles_t * r.tiles_e * r.S * (16 * r.mb) * kFusedTN * 4;
  return (int64_t)r.S * tokens * experts * 4;
}

}  // namespace

extern "C" int64_t hda_router_workspace_bytes(int32_t tokens, int32_t experts, int32_t hidden) {
  if (tokens < 1 || experts < 1 || hidden < kStepK || hidden % kStepK) return -1;
  return ws_bytes(router_shape(tokens, experts, hidden), tokens, experts);
}

extern "C" int hda_router_split_weights(const float* w, int64_t n, void* w_hi, void* w_lo,
                                        void* stream) {
  if (!w || !w_hi || !w_lo || n < 1) return HDA_ERR_INVALID_ARG;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return HDA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(hda_router_split_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), w, static_cast<uint16_t*>(w_hi),
                     static_cast<uint16_t*>(w_lo), n);
  return hipGetLastError() == hipSuccess ? HDA_OK : HDA_ERR_HIP;
}

extern "C" int hda_router_gemm(const void* x, const void* w_hi, const void* w_lo, int32_t tokens,
                               int32_t experts, int32_t hidden, float* out, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  if (!x || !w_hi || !w_lo || !out || tokens < 1 || experts < 1 || hidden < 1)
    return HDA_ERR_INVALID_ARG;
  if (hidden % kStepK) return HDA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_hi) || !aligned16(w_lo)) return HDA_ERR_INVALID_ARG;
  if ((int64_t)tokens * hidden * 2 > 0x7fffffffLL || (int64_t)experts * hidden * 2 > 0x7fffffffLL)
    return HDA_ERR_UNSUPPORTED;                 // 32-bit buffer offsets
  const RouterShape r = router_shape(tokens, experts, hidden);
  const int64_t need = hda_router_workspace_bytes(tokens, experts, hidden);
  if (need > 0 && (!workspace || workspace_bytes < need)) return HDA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return HDA_ERR_INVALID_ARG;
  RouterArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w_hi = static_cast<const uint16_t*>(w_hi);
  a.w_lo = static_cast<const uint16_t*>(w_lo);
  a.out = out;
  a.part = static_cast<float*>(workspace);
  a.T = tokens;
  a.E = experts;
  a.H = hidden;
  a.k_per_wg = r.k_per_wg;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (r.gemv) {
    const dim3 g((unsigned)experts);
    const dim3 b(kGemvThreadsDefault);
    if (r.gemv == 1) hipLaunchKernelGGL((hda_router_gemv_kernel<1, 1>), g, b, 0, hs, a);
    else if (r.gemv == 2) hipLaunchKernelGGL((hda_router_gemv_kernel<2, 1>), g, b, 0, hs, a);
    else if (r.gemv == 4) hipLaunchKernelGGL((hda_router_gemv_kernel<4, 1>), g, b, 0, hs, a);
    else hipLaunchKernelGGL((hda_router_gemv_kernel<8, 1>), g, b, 0, hs, a);
    return hipGetLastError() == hipSuccess ? HDA_OK : HDA_ERR_HIP;
  }
  const dim3 grid(r.tiles_t, r.tiles_e, r.S);
  if (r.fused) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    unsigned long long* cnt = reinterpret_cast<unsigned long long*>(ws);
    float* part = r.S > 1 ? reinterpret_cast<float*>(ws + fused_counter_bytes(r)) : nullptr;
    if (r.mb == 1)
      hipLaunchKernelGGL(hda_router_fused_kernel<1>, grid, dim3(64 * kWaves), 0, hs, a, part, cnt);
    else if (r.mb == 2)
      hipLaunchKernelGGL(hda_router_fused_kernel<2>, grid, dim3(64 * kWaves), 0, hs, a, part, cnt);
    else
      hipLaunchKernelGGL(hda_router_fused_kernel<4>, grid, dim3(64 * kWaves), 0, hs, a, part, cnt);
    return hipGetLastError() == hipSuccess ? HDA_OK : HDA_ERR_HIP;
  }
  if (r.big)
    hipLaunchKernelGGL(hda_router_gemm_lds_kernel, grid, dim3(64 * kBigWaves), 0, hs, a);
  else if (r.mb == 2)
    hipLaunchKernelGGL(hda_router_gemm_kernel<2>, grid, dim3(64 * kWaves), 0, hs, a);
  else
    hipLaunchKernelGGL(hda_router_gemm_kernel<4>, grid, dim3(64 * kWaves), 0, hs, a);
  if (hipGetLastError() != hipSuccess) return HDA_ERR_HIP;
  if (r.S > 1) {
    const int64_t n = (int64_t)tokens * experts;
    const dim3 g((unsigned)((n + 255) / 256));
    if (r.S > 16)
      hipLaunchKernelGGL(hda_router_reduce_kernel<64>, g, dim3(256), 0, hs, a.part, out, n, r.S);
    else
      hipLaunchKernelGGL(hda_router_reduce_kernel<16>, g, dim3(256), 0, hs, a.part, out, n, r.S);
    if (hipGetLastError() != hipSuccess) return HDA_ERR_HIP;
  }
  return HDA_OK;
}

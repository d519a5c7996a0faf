// The rollout-decode linear layer: y_p = s_g,p * W_hat_p h + lambda_p * B_p (A_p h), h = AQN-RMSNorm(x).
//
// "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops" (technical review):
//   §2.1 forward map y = W_hat x + lambda B (A x) with a frozen quantized base and trainable A, B;
//   §3.1 W_hat = s_g * s_b * q (NVFP4); §3.2 decode reads large packed weights for few tokens, so unpack, scale
//   and conversion must keep up with the byte stream; §5.1 AQN-RMSNorm feeds the projections that share its input.
//
// Two kernels per call (three when many tokens share a norm), all on the caller's stream:
//   P  k_prologue  workgroup (token tile of 16, k-chunk, 32-rank LoRA chunk): RMSNorm statistics of its 16 tokens
//                  (one wave per token, in the summation order of the standalone norm, so h is bit-identical to it),
//                  h = bf16(x * rstd * (gamma + sigma * noise)) (or h = x) over its k-chunk, the MFMA B-fragments of h
//                  as f16 scaled by 2^p per (token, 128-wide k-tile) (exact: bf16 has 8 significant bits, f16 11, and
//                  the scale puts the tile's largest magnitude in [2^14, 2^15), so every element above 2^-32 of it
//                  converts exactly), and the chunk's LoRA-down partial t_c = A[:, chunk] h[chunk] with bf16
//                  16x16x32 MFMAs, stored where the LoRA-up MFMA's B-fragments want it.
//   (k_rstd)       with 256 or more tokens the statistics are computed once per token by a kernel of their own and
//                  read by the prologue workgroups instead of recomputed by each.
//   L  k_linear    streams the tiled NVFP4 weight once: per lane one 16-byte load of codes (32 weights) and one dword
//                  of block scales per 128-wide k-tile; FP4 -> f16 with the hardware converter (scale 2^8), times the
//                  E4M3 scale reinterpreted as f16 (byte << 7 is the E4M3 value * 2^-8, exact for normals and
//                  subnormals) gives s_b * q exactly in f16; f16 16x16x32 MFMAs over the tile, whose f32 result is
//                  scaled by the tile's 2^-p (exact) and added to the f32 accumulator. Waves split k; partials meet in
//                  LDS. The LoRA term: the chunk partials of t are summed in chunk order (results do not depend on
//                  scheduling) and split t = t_hi + t_lo, both bf16 (t - t_hi is exact in f32, 16 significant bits
//                  kept); B t is then two bf16 MFMAs per row group. The epilogue applies s_g, lambda, residual,
//                  SiLU(gate) * up, broadcast and rounding. Everything it reads is fetched before the weight stream.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <hip/hip_ext.h>
#include <mutex>
#include <type_traits>

#include "qn_device.hpp"
#include "qn_norm.hpp"

namespace qn {
namespace {

constexpr int kMaxProj = 4;
constexpr int kMaxRank = 64;
constexpr int kRankChunks = kMaxRank / 32;  // 32-wide rank chunks of the LoRA-up MFMA
constexpr int kMaxPg = kMaxProj * kRankChunks;
constexpr int kMaxTokensPerLaunch = 128;
constexpr int kMaxChunkTiles = 8;           // k-tiles per prologue chunk (h of the chunk is staged in LDS)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct ProjArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* s_g;
  const uint16_t* A;
  const uint16_t* B;
  void* y;
  const uint16_t* res;
  int64_t n, ldy, ld_res;
  int32_t r, y_dtype, y_repeat, head_dim;
  float lambda;
  int32_t rg_begin;  // first row group of this projection in the launch's flattened list
};

// Store one output value (f32 or bf16) at element (token row tok_off = token * ldy, column n) and, with a GQA
// broadcast (y_repeat > 1), at the same position of each of the y_repeat copies of its head: copy g of head h sits
// at column (h * y_repeat + g) * head_dim + n % head_dim. The head split is taken once (32-bit: n < 2^31), the
// copies are head_dim apart.
__device__ __forceinline__ void store_output(void* y, int32_t y_dtype, int64_t tok_off, int64_t n, int32_t y_repeat,
                                             int32_t head_dim, float out) {
  int64_t off = tok_off + n, step = 0;
  int rep = 1;
  if (y_repeat > 1) {
    const uint32_t h = (uint32_t)n / (uint32_t)head_dim, d = (uint32_t)n - h * (uint32_t)head_dim;
    off = tok_off + (int64_t)h * y_repeat * head_dim + d;
    step = head_dim;
    rep = y_repeat;
  }
  if (y_dtype == QN_F32) {
    float* const p = reinterpret_cast<float*>(y) + off;
    for (int g = 0; g < rep; ++g) p[g * step] = out;
  } else {
    uint16_t* const p = reinterpret_cast<uint16_t*>(y) + off;
    const uint16_t v = f32_to_bf16(out);
    for (int g = 0; g < rep; ++g) p[g * step] = v;
  }
}

struct LinearArgs {
  ProjArgs p[kMaxProj];
  int32_t nproj, epilogue;
  int64_t m, k, kp;
  int64_t tok0;            // first token of this launch
  const u32x4* xs;         // activation fragments, [tile][kp/128][4][64] x 16 bytes
  const float* xsc;        // [tile][kp/128][16] 2^-p per (token, k-tile)
  const u32x4* t_part;     // LoRA-down partials, [nproj][tile][kRankChunks][ks][64 lanes][8 f32]
  int64_t t_bytes;
  int32_t ks;              // LoRA-down k-chunks
};

// Workspace carve-up (256-byte aligned regions).
struct Workspace {
  size_t xs, xsc, rstd, tok_p, t_part, t_fin, pbuf, t_fused, cnt, xmx, total;
};
constexpr int kMxScStage = 64 * 16 * 4;  // activation E8M0 words of one (128-token block, k-tile): [lane][tile][hi, lo]

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Prologue k-chunks: at most 8 where possible, each a whole number of k-tiles, at most kMaxChunkTiles of them. The
// chunking depends on k alone, so a call with the norm and one fed the standalone norm's output sum the LoRA-down
// partials in the same order.
inline int64_t chunk_tiles(int64_t KT) {
  const int64_t ct = ceil_div(KT, 8);
  return ct < kMaxChunkTiles ? ct : kMaxChunkTiles;
}
inline int64_t lora_chunks(int64_t k) {
  const int64_t KT = ceil_div(k, kKTile);
  return ceil_div(KT, chunk_tiles(KT));
}

// Control words of the workspace, zero between calls: 256 split-k arrival counters, then the fused decode kernel's
// consumer counter (kCountWords in all; every call that runs the prologue zeroes them), then the prologue's own
// arrival counters for summing the LoRA-down t (kTsumWords: one per pair group and token tile of up to 64 tokens;
// each is reset by the last workgroup to arrive). The fused kernel's LoRA-down partials (kFusedItemsMax items) are
// zero between calls too: they are their own ready flags.
constexpr int kFusedItemsMax = 192;
constexpr int kCountWords = 256 + 1;
constexpr int kTsumWords = 4 * 2 * 4;  // kMaxPg x token tiles (kMaxPg = kMaxProj * kRankChunks)
constexpr int kCoherent = 16;          // buffer-access cache policy sc1: device-coherent, past the XCD's L2

struct Opts;
size_t gemv_pbuf_bytes(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj, const Opts& o);

// mx: a call of mxfp4_lora_linear (the scaled-MFMA kernel at every token count: t summed for every token tile, and the
// activations' block scales).
Workspace workspace_layout(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj, const Opts& o, bool mx = false) {
  const int64_t KT = ceil_div(k, kKTile), kp = KT * kKTile;
  const int64_t mp = ceil_div(m, 16) * 16;
  Workspace w;
  size_t off = 0;
  // Regions that must be zero between calls come first, at the same offsets in every call's layout, so that no other
  // call sharing the workspace (with other shapes, hence other offsets for its data) writes over them.
  w.cnt = off;     off = align256(off + (kCountWords + kTsumWords) * 4);  // (see kCountWords)
  w.t_fused = off; off = align256(off + (size_t)kFusedItemsMax * kWave * 8 * 4);
  w.xs = off;     off = align256(off + (size_t)mp * kp * 2);
  w.xsc = off;    off = align256(off + (size_t)mp * KT * 4);
  w.rstd = off;   off = align256(off + (size_t)mp * 4);
  w.tok_p = off;  off = align256(off + (size_t)mp * 4);
  w.t_part = off; off = align256(off + (size_t)nproj * (mp / 16) * kRankChunks * lora_chunks(k) * kWave * 32);
  w.t_fin = off;  off = align256(off + (m > 16 || mx ? (size_t)nproj * (mp / 16) * kRankChunks * 2 * kWave * 16 : 0));
  w.pbuf = off;   off = align256(off + (mx ? 0 : gemv_pbuf_bytes(m, k, projs, nproj, o)));
  w.xmx = off;    off = align256(off + (mx ? (size_t)ceil_div(mp, 128) * KT * kMxScStage : 0));
  w.total = off;
  return w;
}

// ------------------------------------------------------------------------------------------------------------------
// P: prologue. Workgroup (token tile, k-chunk c of CT k-tiles, pair group pg = one 32-rank chunk jc of projection p);
// 16 waves. Every pair group of a chunk computes the same h; pair group 0 stores the MFMA fragments and tile scales.
constexpr int kProWaves = 16;

struct PrologueArgs {
  const uint16_t* x;
  int64_t ldx, m, k, KT;
  int32_t CT, ks, npg, has_aqn, nproj;
  int32_t vec_x, vec_g, vec_z;
  const uint16_t* gamma;
  const float* noise;
  int64_t noise_ld;
  float sigma, eps;
  const float* rstd_in;   // statistics from k_rowstats, or null: computed here
  const int32_t* tok_p;   // per-token exponents p from k_rowstats (2^p for every k-tile of the token), or null
  const uint16_t* A[kMaxProj];
  int32_t r[kMaxProj];
  int8_t pg_p[kMaxPg], pg_jc[kMaxPg];
  u32x4* xs;
  float* xsc;
  float* t_part;
  uint32_t* cnt;  // arrival counters of the linear kernel, zeroed here
  int32_t ncnt;
  u32x4* t_fin;       // or null: the last workgroup of each (pair group, token tile) also sums the LoRA-down chunk
  uint32_t* t_cnt;    // partials into bf16 hi/lo fragments ([p][tile][jc][hi, lo][lane]); t_cnt: their arrivals
  uint32_t* xmx_sc;  // non-null: activations out as E4M3 hi and lo parts with E8M0 scales (the scaled-MFMA kernel)
  int32_t tgs;    // tokens per workgroup: 16 (a whole token tile) or 4 (the tile split over four workgroups)
  int32_t pgm;    // pair groups per workgroup: 1, or 2 (h computed once for both, many tokens)
  QnDraw draw;    // noise drawn on the device (draw.on) instead of read from `noise`
};

// Sum of squares of one row by one wave, in the summation order of the standalone norm with NT threads (as
// row_sumsq_one_wave), read through a buffer descriptor: row_off is the row's byte offset in it. VEC: 16-byte loads.
// The first batch of loads (eight chunks per lane) is issued separately by row_sumsq_load, ahead of other loads, so
// the sum waits for the row alone.
template <int NT>
struct RowSqPlan {
  static constexpr int V = NT / kWave;  // stand-in threads per lane
  static constexpr int VB = V < 8 ? V : 8;
  static constexpr int IB = 8 / VB;
};

template <bool VEC>
__device__ __forceinline__ void bload_chunk(rsrc_t src, uint32_t off, uint32_t (&w)[4]) {
  if (VEC) {
    const u32x4 q = bload16(src, off);
    w[0] = q[0]; w[1] = q[1]; w[2] = q[2]; w[3] = q[3];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(src, off == kOutOfRange ? off : off + 4 * e, 0, 0);
      const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(src, off == kOutOfRange ? off : off + 4 * e + 2, 0, 0);
      w[e] = lo | (hi << 16);
    }
  }
}

template <int NT, bool VEC>
__device__ __forceinline__ void row_sumsq_load(rsrc_t src, uint32_t row_off, int d, uint32_t (&q)[8][4]) {
  using P = RowSqPlan<NT>;
  const int lane = threadIdx.x % kWave, nch = d / 8;
#pragma unroll
  for (int ib = 0; ib < P::IB; ++ib)
#pragma unroll
    for (int vb = 0; vb < P::VB; ++vb) {
      const int ch = ib * NT + vb * kWave + lane;
      bload_chunk<VEC>(src, ch < nch ? row_off + (uint32_t)ch * 16 : kOutOfRange, q[ib * P::VB + vb]);
    }
}

template <int NT, bool VEC>
__device__ inline float row_sumsq_buf(rsrc_t src, uint32_t row_off, int d, const uint32_t (&pre)[8][4]) {
  using P = RowSqPlan<NT>;
  constexpr int V = P::V, VB = P::VB, IB = P::IB;
  const int lane = threadIdx.x % kWave;
  const int nch = d / 8;
  float ss[V];
#pragma unroll
  for (int v = 0; v < V; ++v) ss[v] = 0.0f;
  for (int i0 = 0; i0 * NT < nch; i0 += IB) {
#pragma unroll
    for (int v0 = 0; v0 < V; v0 += VB) {
      uint32_t q[IB][VB][4];
      if (i0 == 0 && v0 == 0) {
#pragma unroll
        for (int ib = 0; ib < IB; ++ib)
#pragma unroll
          for (int vb = 0; vb < VB; ++vb)
#pragma unroll
            for (int e = 0; e < 4; ++e) q[ib][vb][e] = pre[ib * VB + vb][e];
      } else {
#pragma unroll
        for (int ib = 0; ib < IB; ++ib)
#pragma unroll
          for (int vb = 0; vb < VB; ++vb) {
            const int ch = (i0 + ib) * NT + (v0 + vb) * kWave + lane;
            bload_chunk<VEC>(src, ch < nch ? row_off + (uint32_t)ch * 16 : kOutOfRange, q[ib][vb]);
          }
      }
      // each stand-in adds its chunks in chunk order, elements in order
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
          if ((i0 + ib) * NT + (v0 + vb) * kWave + lane >= nch) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = lo_bf16(q[ib][vb][e]), x1 = hi_bf16(q[ib][vb][e]);
            ss[v0 + vb] = __fadd_rn(ss[v0 + vb], __fmul_rn(x0, x0));
            ss[v0 + vb] = __fadd_rn(ss[v0 + vb], __fmul_rn(x1, x1));
          }
        }
    }
  }
  float tot = 0.0f;
#pragma unroll
  for (int v = 0; v < V; ++v) tot = __fadd_rn(tot, wave_sum(ss[v]));
  return tot;
}

// Eight consecutive bf16 (VEC: one 16-byte load) and eight f32 (two loads) through a buffer descriptor.
template <bool VEC>
__device__ __forceinline__ void bload_bf16x8(rsrc_t src, uint32_t off, uint32_t (&w)[4]) {
  bload_chunk<VEC>(src, off, w);
}
template <bool VEC>
__device__ __forceinline__ void bload_f32x8(rsrc_t src, uint32_t off, float (&z)[8]) {
  if (VEC) {
    const f32x4 z0 = __builtin_bit_cast(f32x4, bload16(src, off));
    const f32x4 z1 = __builtin_bit_cast(f32x4, bload16(src, off == kOutOfRange ? off : off + 16));
#pragma unroll
    for (int e = 0; e < 4; ++e) { z[e] = z0[e]; z[4 + e] = z1[e]; }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      z[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(src, off == kOutOfRange ? off : off + 4 * e, 0, 0));
  }
}

// Power-of-two scale exponent of a group of bf16 values with largest magnitude amax: amax * 2^p in [2^14, 2^15), read
// off the exponent field and kept within the normal range so 2^p and 2^-p are plain f32 powers of two.
__device__ __forceinline__ int act_exponent(float amax) {
  int pw = 0;
  if (amax > 0.0f) {
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127;
    pw = 14 - (e < -126 ? -126 : e);
    pw = pw > 126 ? 126 : pw;
  }
  return pw;
}

// E8M0 exponent s of a 32-value block with largest magnitude amax for the scaled-MFMA activations: amax * 2^-s in
// [128, 256), so every value of the block lies within the E4M3 range after the scaling; 0 for a block of zeros.
__device__ __forceinline__ int mx_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127;
  const int s = e - 7;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}


// Row statistics for many tokens: one wave per token. With the norm, rstd in the summation order of the standalone
// norm; then the token's largest |h| over its whole row (h exactly as the prologue computes it), giving one exponent
// p per token for all its k-tiles.
template <int NT, bool AQN, bool VEC>
__global__ void __launch_bounds__(16 * kWave) k_rowstats(PrologueArgs a, float* __restrict__ rstd_out,
                                                         int32_t* __restrict__ p_out) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int tile = blockIdx.x, k = (int)a.k, m = (int)a.m;
  const int rows = m - tile * 16 < 16 ? m - tile * 16 : 16;
  if (wave >= rows) return;
  const rsrc_t xsrc = make_rsrc(a.x + (int64_t)tile * 16 * a.ldx, ((int64_t)(rows - 1) * a.ldx + k) * 2);
  const rsrc_t gsrc = make_rsrc(a.gamma, AQN ? (int64_t)k * 2 : 0);
  const int64_t nld = a.noise_ld;
  const rsrc_t zsrc = make_rsrc(a.noise ? a.noise + (int64_t)tile * 16 * nld : nullptr,
                                (AQN && a.noise) ? ((int64_t)(rows - 1) * nld + k) * 4 : 0);
  const uint32_t row = (uint32_t)((int64_t)wave * a.ldx * 2);
  float rstd = 0.f;
  if (AQN) {
    uint32_t sq[8][4];
    row_sumsq_load<NT, VEC>(xsrc, row, k, sq);
    rstd = rms_rstd(row_sumsq_buf<NT, VEC>(xsrc, row, k, sq), k, a.eps);
  }
  float amax = 0.f;
  const int nch = k / 8;
  for (int c0 = 0; c0 < nch; c0 += 4 * kWave) {
    uint32_t hx[4][4], hg[4][4];
    float hz[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * kWave + lane;
      bload_bf16x8<VEC>(xsrc, c < nch ? row + (uint32_t)c * 16 : kOutOfRange, hx[u]);
      if (AQN) {
        bload_bf16x8<VEC>(gsrc, c < nch ? (uint32_t)c * 16 : kOutOfRange, hg[u]);
        if (!a.draw.on) bload_f32x8<VEC>(zsrc, c < nch ? (uint32_t)((wave * nld + c * 8) * 4) : kOutOfRange, hz[u]);
      }
    }
    if (AQN && a.draw.on) {
      // drawn noise of this token's chunks, computed while the loads are in flight
      const uint64_t r = draw_index(a.draw, (int64_t)tile * 16 + wave);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < nch) aqn_noise8(a.draw, r, (uint64_t)c, hz[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (c0 + u * kWave + lane >= nch) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lo = hx[u][e] & 0xffffu, hi = hx[u][e] >> 16;
        if (AQN) {
          lo = aqn_value(lo_bf16(hx[u][e]), rstd, (uint16_t)hg[u][e], hz[u][2 * e], a.sigma);
          hi = aqn_value(hi_bf16(hx[u][e]), rstd, (uint16_t)(hg[u][e] >> 16), hz[u][2 * e + 1], a.sigma);
        }
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(lo << 16)), fabsf(__uint_as_float(hi << 16))));
      }
    }
  }
  amax = wave_max(amax);
  if (lane == 0) {
    const int64_t tok = (int64_t)tile * 16 + wave;
    if (AQN) rstd_out[tok] = rstd;
    p_out[tok] = act_exponent(amax);
  }
}

// VEC: x rows, gamma and the noise rows start 16-byte aligned at every 8-element group (all loads 16 bytes wide).
template <int NT, bool AQN, bool VEC, int PGM>
__global__ void __launch_bounds__(kProWaves * kWave) k_prologue(PrologueArgs a) {
  constexpr int kCT = kMaxChunkTiles;                              // k-tiles per chunk (at most)
  constexpr int kProSlices = kCT * 4 / kProWaves;                // 32-wide k-slices per wave (at most)
  constexpr int kPasses = kCT * 256 / (kProWaves * kWave);        // 8-element groups per thread (at most)
  constexpr int kHRow = kMaxChunkTiles * kKTile + 8;  // LDS row of h (bf16), padded against bank conflicts
  __shared__ float s_rstd[16];
  __shared__ __attribute__((aligned(16))) uint16_t s_h[16][kHRow];
  __shared__ f32x4 s_red[kProWaves][2][kWave];
  __shared__ int s_tlast;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  // workgroup x = (token tile, token group): tokens [tlo, tlo + tgs) of the tile are this workgroup's (their
  // statistics, h, fragments and LoRA-down partials); the other tokens' h stays zero
  const int ngpt = 16 / a.tgs;
  const int tile = blockIdx.x / ngpt, tgrp = blockIdx.x % ngpt, ntiles = gridDim.x / ngpt;
  const int tlo = tgrp * a.tgs;
  auto mine = [&](int t) { return t >= tlo && t < tlo + a.tgs; };
  const int c = blockIdx.y, pz = blockIdx.z;  // pair groups pz * pgm .. + pgm - 1
  const int KT = (int)a.KT, k = (int)a.k, m = (int)a.m;
  const int kt0 = c * a.CT;
  const int ctn = KT - kt0 < a.CT ? KT - kt0 : a.CT;  // k-tiles in this chunk
  const int kc0 = kt0 * kKTile;
  const int rows = m - tile * 16 < 16 ? m - tile * 16 : 16;  // tokens of this tile
  // pair groups -> (projection p, 32-rank chunk jc), from the adapter ranks (constant-index argument reads)
  constexpr int kPgm = PGM;  // pair groups per workgroup (at most)
  int pgp[kPgm], pgjc[kPgm], pgr[kPgm];
  const uint16_t* pgA[kPgm];
#pragma unroll
  for (int gi = 0; gi < kPgm; ++gi) {
    const int pg = pz * a.pgm + gi;
    int p = -1, jc = 0, base = 0, r = 0;
    const uint16_t* Ap = nullptr;
#pragma unroll
    for (int q = 0; q < kMaxProj; ++q) {
      const int nq = q < a.nproj ? (a.r[q] + 31) / 32 : 0;
      if (gi < a.pgm && p < 0 && pg < base + nq) {
        p = q;
        jc = pg - base;
        Ap = a.A[q];
        r = a.r[q];
      }
      base += nq;
    }
    pgp[gi] = p;
    pgjc[gi] = jc;
    pgr[gi] = r;
    pgA[gi] = Ap;
  }
  const bool lora = pgp[0] >= 0;
  if (tile == 0 && tgrp == 0 && c == 0 && pz == 0 && (int)threadIdx.x < a.ncnt) a.cnt[threadIdx.x] = 0u;

  // Loads, in the order they are needed (each wait then covers its own loads only): the first batch of the
  // statistics row, the inputs of h, the LoRA-down A fragments.
  const rsrc_t xsrc = make_rsrc(a.x + (int64_t)tile * 16 * a.ldx, ((int64_t)(rows - 1) * a.ldx + k) * 2);
  // statistics: wave w <-> token w ^ 8 of the tile. The h groups of a token lie in the waves from about its own
  // index on (one wave per token at 4 k-tiles per chunk), so the waves that sum a workgroup's rows are not the ones
  // that draw its noise (with a seeded draw) and the two run side by side.
  const int st = wave ^ 8;
  const bool own_stats = AQN && !a.rstd_in && st < rows && mine(st);
  const uint32_t stats_row = (uint32_t)((int64_t)st * a.ldx * 2);
  uint32_t sq[8][4];
  if (AQN) row_sumsq_load<NT, VEC>(xsrc, own_stats ? stats_row : kOutOfRange, own_stats ? k : 0, sq);

  // inputs of h for this thread's 8-element groups (x, and gamma and noise with the norm). Group g: token
  // g / (ctn*16), k-tile (g % (ctn*16)) / 16 of the chunk; the 16 groups of one (token, k-tile) are 16 consecutive
  // lanes.
  const rsrc_t gsrc = make_rsrc(a.gamma, AQN ? (int64_t)k * 2 : 0);
  const int64_t nld = a.noise_ld;
  const rsrc_t zsrc = make_rsrc(a.noise ? a.noise + (int64_t)tile * 16 * nld : nullptr,
                                (AQN && a.noise) ? ((int64_t)(rows - 1) * nld + k) * 4 : 0);
  const int ngroups = 16 * ctn * 16;  // a multiple of 256: a wave is either wholly in range or wholly out
  uint32_t hx[kPasses][4], hg[kPasses][4];
  float hz[kPasses][8];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int g = threadIdx.x + ps * kProWaves * kWave;
    const int t = g / (ctn * 16), kg = g % (ctn * 16);
    const int kk = kc0 + kg * 8;
    const bool ok = g < ngroups && t < rows && kk < k && mine(t);
    bload_bf16x8<VEC>(xsrc, ok ? (uint32_t)(((int64_t)t * a.ldx + kk) * 2) : kOutOfRange, hx[ps]);
    if (AQN) {
      bload_bf16x8<VEC>(gsrc, ok ? (uint32_t)kk * 2 : kOutOfRange, hg[ps]);
      if (!a.draw.on) bload_f32x8<VEC>(zsrc, ok ? (uint32_t)((t * nld + kk) * 4) : kOutOfRange, hz[ps]);
    }
  }

  // LoRA-down A fragments of this wave's slices, issued last (needed last). Fragment (g, slice s): ranks
  // jc*32 + g*16 + lane%16, k = kc0 + 32 s + 8 (lane/16) .. + 8; ranks past r and k past the row read as 0.
  const int nsl = ctn * 4;
  u32x4 af[kPgm][2][kProSlices];
#pragma unroll
  for (int gi = 0; gi < kPgm; ++gi) {
    const int jc = pgjc[gi], r = pgr[gi];
    const rsrc_t asrc = make_rsrc(pgA[gi], pgp[gi] >= 0 ? (int64_t)r * k * 2 : 0);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < kProSlices; ++i) {
        const int s = wave + i * kProWaves;
        const int j = jc * 32 + g * 16 + lane % 16;
        const int kk = kc0 + s * 32 + (lane / 16) * 8;
        const bool ok = pgp[gi] >= 0 && s < nsl && j < r && kk < k;
        af[gi][g][i] = bload16(asrc, ok ? (uint32_t)(((int64_t)j * k + kk) * 2) : kOutOfRange);
      }
  }

  // drawn noise of this thread's groups, computed while the loads above are in flight
  if (AQN && a.draw.on) {
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int g = threadIdx.x + ps * kProWaves * kWave;
      const int t = g / (ctn * 16), kg = g % (ctn * 16);
      const int kk = kc0 + kg * 8;
      if (g < ngroups && t < rows && kk < k && mine(t)) {
        aqn_noise8(a.draw, draw_index(a.draw, (int64_t)tile * 16 + t), (uint64_t)(kk / 8), hz[ps]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) hz[ps][e] = 0.0f;  // as an out-of-range load would give (h of x = 0 stays 0)
      }
    }
  }

  // statistics of token st = wave ^ 8 (every token of the tile has exactly one wave)
  if (AQN) {
    float rstd = 0.f;
    if (st < rows && mine(st))
      rstd = a.rstd_in ? gload(a.rstd_in + tile * 16 + st)
                       : rms_rstd(row_sumsq_buf<NT, VEC>(xsrc, stats_row, k, sq), k, a.eps);
    if (lane == 0) s_rstd[st] = rstd;
  }
  __syncthreads();

  // h, its LDS copy for the LoRA-down, and (pair group 0) the f16 fragments and tile scales
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int g = threadIdx.x + ps * kProWaves * kWave;
    if (g >= ngroups) break;
    const int t = g / (ctn * 16), kg = g % (ctn * 16), ktl = kg / 16, jj = kg % 16;
    uint32_t hv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) hv[e] = hx[ps][e];
    if (AQN) {
      const float rstd = s_rstd[t];
      const int64_t tok = tile * 16 + t, kk = kc0 + (int64_t)kg * 8;
      if (tok < a.m && kk < a.k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = aqn_value(lo_bf16(hv[e]), rstd, (uint16_t)hg[ps][e], hz[ps][2 * e], a.sigma);
          const uint32_t hi = aqn_value(hi_bf16(hv[e]), rstd, (uint16_t)(hg[ps][e] >> 16), hz[ps][2 * e + 1], a.sigma);
          hv[e] = lo | (hi << 16);
        }
      }
    }
    *reinterpret_cast<u32x4*>(&s_h[t][kg * 8]) = u32x4{hv[0], hv[1], hv[2], hv[3]};
    if (pz == 0 && a.xmx_sc) {
      // scaled-MFMA activations: each 32-value block (4 consecutive lanes) as hi = E4M3(h * 2^-s_hi) and
      // lo = E4M3((h - hi * 2^s_hi) * 2^-s_lo), both with E8M0 block exponents; in the 16x16x128 B-operand layout
      // (lane (k / 16) % 4 * 16 + token holds k % 16 + (k / 64) * 16 of its 32 bytes), the scale of block b in lane
      // b * 16 + token. The 8 values of this thread are one contiguous 8-byte piece of a lane.
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = lo_bf16(hv[e]);
        v[2 * e + 1] = hi_bf16(hv[e]);
      }
      float am = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
      am = fmaxf(am, __shfl_xor(am, 1, kWave));
      am = fmaxf(am, __shfl_xor(am, 2, kWave));
      const int sh = mx_block_exp(am);
      // (v_cvt_pk_fp8_f32: two f32 to OCP E4M3, round to nearest even; every scaled value lies within 256, so
      // nothing saturates)
      const float dh = ldexpf(1.0f, -sh), uh = ldexpf(1.0f, sh);  // (2^-127 is subnormal: no exponent-field trick)
      uint32_t hb[2] = {0u, 0u}, lb[2] = {0u, 0u};
      float rr[8], ar = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[2 * e] * dh, v[2 * e + 1] * dh, 0, false);
        hb[e / 2] |= ((uint32_t)pk & 0xFFFFu) << (16 * (e % 2));
        // the remainders, exact: v has 8 significant bits and hi * 2^s_hi its leading ones
        rr[2 * e] = v[2 * e] - __builtin_amdgcn_cvt_f32_fp8(pk, 0) * uh;
        rr[2 * e + 1] = v[2 * e + 1] - __builtin_amdgcn_cvt_f32_fp8(pk, 1) * uh;
        ar = fmaxf(ar, fmaxf(fabsf(rr[2 * e]), fabsf(rr[2 * e + 1])));
      }
      ar = fmaxf(ar, __shfl_xor(ar, 1, kWave));
      ar = fmaxf(ar, __shfl_xor(ar, 2, kWave));
      const int sl = mx_block_exp(ar);
      const float dl = ldexpf(1.0f, -sl);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(rr[2 * e] * dl, rr[2 * e + 1] * dl, 0, false);
        lb[e / 2] |= ((uint32_t)pk & 0xFFFFu) << (16 * (e % 2));
      }
      const int64_t kt = kt0 + ktl;
      if (mine(t)) {
        const int L = ((jj / 2) % 4) * 16 + t, bo = (jj / 8) * 16 + (jj % 2) * 8;
        uint8_t* const fb = reinterpret_cast<uint8_t*>(a.xs) + ((tile * a.KT + kt) * 2) * 2048 + L * 32 + bo;
        *reinterpret_cast<u32x2*>(fb) = u32x2{hb[0], hb[1]};
        *reinterpret_cast<u32x2*>(fb + 2048) = u32x2{lb[0], lb[1]};
        if (jj % 4 == 0) {  // [tile block of 8][k-tile][lane][tile % 8][hi, lo] E8M0 words
          uint32_t* const sp = a.xmx_sc + (((int64_t)(tile / 8) * a.KT + kt) * kWave + (jj / 4) * 16 + t) * 16 +
                               (tile % 8) * 2;
          *reinterpret_cast<u32x2*>(sp) = u32x2{(uint32_t)(sh + 127), (uint32_t)(sl + 127)};
        }
      }
    } else if (pz == 0) {
      // tile amax over the 16 lanes of this (token, k-tile), then 2^p with amax * 2^p in [2^14, 2^15), read off the
      // exponent field and kept within the normal range so 2^p and 2^-p are plain f32 powers of two
      int pw;
      if (a.tok_p) {
        pw = t < rows ? gload(a.tok_p + tile * 16 + t) : 0;  // one exponent per token (many-token path)
      } else {
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(hv[e])), fabsf(hi_bf16(hv[e]))));
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
        pw = act_exponent(amax);
      }
      const float up = __uint_as_float((uint32_t)(pw + 127) << 23);
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f16x2 v;
        v[0] = (_Float16)__fmul_rn(lo_bf16(hv[e]), up);
        v[1] = (_Float16)__fmul_rn(hi_bf16(hv[e]), up);
        packed[e] = __builtin_bit_cast(uint32_t, v);
      }
      const int64_t kt = kt0 + ktl;
      const int s = jj / 4, lhi = jj % 4;
      if (mine(t)) {
        a.xs[((tile * a.KT + kt) * 4 + s) * kWave + lhi * 16 + t] = u32x4{packed[0], packed[1], packed[2], packed[3]};
        if (jj == 0) a.xsc[(tile * a.KT + kt) * 16 + t] = __uint_as_float((uint32_t)(127 - pw) << 23);
      }
    }
  }
  __syncthreads();
  if (!lora) return;

  // LoRA-down over the chunk, per pair group: B-fragment (token lane%16, k = 32 s + 8 (lane/16) .. + 8) from LDS
#pragma unroll
  for (int gi = 0; gi < kPgm; ++gi) {
    const int p = pgp[gi], jc = pgjc[gi];
    if (p < 0) break;
    if (gi > 0) __syncthreads();  // the previous group's reduction is done with s_red
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < kProSlices; ++i) {
      const int s = wave + i * kProWaves;
      if (s >= nsl) break;
      const u32x4 b = *reinterpret_cast<const u32x4*>(&s_h[lane % 16][s * 32 + (lane / 16) * 8]);
#pragma unroll
      for (int g = 0; g < 2; ++g)
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[gi][g][i]),
                                                         __builtin_bit_cast(bf16x8, b), acc[g], 0, 0, 0);
    }
    mfma_settle(acc[0]);  // (the loop's exit separates the MFMAs from these stores)
    mfma_settle(acc[1]);
    s_red[wave][0][lane] = acc[0];
    s_red[wave][1][lane] = acc[1];
    __syncthreads();
    if (threadIdx.x < 512) {
      // thread (rank group g, rank row jr, token column tc); D lane (jr/4)*16 + tc, element jr%4; waves in order
      const int g = threadIdx.x / 256, jr = (threadIdx.x % 256) / 16, tc = threadIdx.x % 16;
      const int src = (jr / 4) * 16 + tc, q = jr % 4;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kProWaves; ++w) v += s_red[w][g][src][q];
      const int jl = g * 16 + jr;  // rank within the 32-rank chunk
      const int L = (jl / 8) * 16 + tc;
      float* const dst = a.t_part + ((((int64_t)p * ntiles + tile) * kRankChunks + jc) * a.ks + c) * kWave * 8 + L * 8 +
                         jl % 8;
      if (mine(tc)) {
        if (a.t_fin) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // read back below
        else *dst = v;
      }
    }
  }

  // With t_fin (one pair group per workgroup): the last of the ks * ngpt workgroups of this (pair group, token tile)
  // to arrive adds the chunk partials in chunk order (the order of every other reader of them) and stores t as bf16
  // hi and lo B-fragments. The partials were written with device-scope stores that completed before the arrival and
  // are read with device-coherent loads, so no cache-wide fence is needed. Waves 0 and 1 take ranks 0-3 and 4-7 of
  // each lane's eight.
  if (PGM == 1 && a.t_fin) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t* const ctr = a.t_cnt + pz * ntiles + tile;
    if (threadIdx.x == 0)
      s_tlast = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(a.ks * ngpt - 1);
    __syncthreads();
    if (s_tlast && wave < 2) {
      const int p = pgp[0], jc = pgjc[0];
      const int64_t slot = ((int64_t)p * ntiles + tile) * kRankChunks + jc;
      const rsrc_t src = make_rsrc(a.t_part + slot * a.ks * kWave * 8, (int64_t)a.ks * kWave * 8 * 4);
      constexpr int kB = 16;  // chunk partials loaded together
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < a.ks; c0 += kB) {
        u32x4 q[kB];
#pragma unroll
        for (int v = 0; v < kB; ++v)
          q[v] = __builtin_amdgcn_raw_buffer_load_b128(
              src, c0 + v < a.ks ? (uint32_t)((((c0 + v) * kWave + lane) * 8 + wave * 4) * 4) : kOutOfRange, 0,
              kCoherent);
#pragma unroll
        for (int v = 0; v < kB; ++v)
          if (c0 + v < a.ks) t = (c0 + v == 0) ? __builtin_bit_cast(f32x4, q[v]) : t + __builtin_bit_cast(f32x4, q[v]);
      }
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t th = f32_to_bf16(t[e]);
        const uint32_t tl = f32_to_bf16(t[e] - bf16_to_f32((uint16_t)th));  // t - th is exact in f32
        if (e % 2 == 0) {
          hi[e / 2] = th;
          lo[e / 2] = tl;
        } else {
          hi[e / 2] |= th << 16;
          lo[e / 2] |= tl << 16;
        }
      }
      uint32_t* const d = reinterpret_cast<uint32_t*>(a.t_fin + slot * 2 * kWave + lane) + wave * 2;
      *reinterpret_cast<u32x2*>(d) = u32x2{hi[0], hi[1]};
      *reinterpret_cast<u32x2*>(d + kWave * 4) = u32x2{lo[0], lo[1]};
      if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------------------------------------------------------
// L: main streaming kernel.
//   TMT  token tiles of 16 in this launch
//   R    row groups (16 rows each) per workgroup; with SILU they are (gate, up) pairs: slot 2i = gate, 2i+1 = up
//   W    waves; wave w takes the contiguous k-tile range [w*KT/W, (w+1)*KT/W) for all R row groups
// Per k-tile and row group a lane loads one 16-byte code chunk and one dword of scales; per token tile and slice one
// 16-byte B-fragment, plus one dword: the 2^-p of the lane's token for this k-tile. Loads of tile i+1 are issued
// before tile i is computed.
template <int TMT, int R>
struct TileBuf {
  u32x4 c[R];
  uint32_t sc[R];
  u32x4 b[TMT][4];
  uint32_t xu[TMT];
};

// Operand streams of one workgroup. Buffer descriptors are wave-uniform (SGPRs); each lane adds one 32-bit offset.
// Dead row-group slots have num_records = 0 and absent tokens an out-of-range offset, so their loads return zeros.
template <int TMT, int R>
struct Streams {
  rsrc_t c[R], s[R], b, x;
  uint32_t c_off, s_off, b_off[TMT], x_off[TMT];
};

template <int TMT, int R>
__device__ __forceinline__ void load_tile(TileBuf<TMT, R>& t, const Streams<TMT, R>& st, int64_t kt) {
  const int kc = __builtin_amdgcn_readfirstlane((int)(kt * kTileCodeBytes));
  const int ks = __builtin_amdgcn_readfirstlane((int)(kt * kTileScaleBytes));
  const int kb = __builtin_amdgcn_readfirstlane((int)(kt * 4 * kWave * 16));
  const int kx = __builtin_amdgcn_readfirstlane((int)(kt * 16 * 4));
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    t.c[rr] = __builtin_amdgcn_raw_buffer_load_b128(st.c[rr], st.c_off, kc, kNonTemporal);
    t.sc[rr] = __builtin_amdgcn_raw_buffer_load_b32(st.s[rr], st.s_off, ks, kNonTemporal);
  }
#pragma unroll
  for (int tt = 0; tt < TMT; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      t.b[tt][q] = __builtin_amdgcn_raw_buffer_load_b128(st.b, st.b_off[tt] + q * kWave * 16, kb, 0);
#pragma unroll
  for (int tt = 0; tt < TMT; ++tt) t.xu[tt] = __builtin_amdgcn_raw_buffer_load_b32(st.x, st.x_off[tt], kx, 0);
}

template <int TMT, int R>
__device__ __forceinline__ void compute_tile(const TileBuf<TMT, R>& t, f32x4 (&acc)[R][TMT]) {
  f32x4 part[R][TMT];
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) part[rr][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const uint32_t sv = ((t.sc[rr] >> (8 * s)) & 0xFFu) * 0x00800080u;  // E4M3 byte << 7 = E4M3 * 2^-8 in f16
      const f16x2 sh = __builtin_bit_cast(f16x2, sv);
      const uint32_t cw = t.c[rr][s];
      const f16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 0) * sh;
      const f16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 1) * sh;
      const f16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 2) * sh;
      const f16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 3) * sh;
      const f16x8 av = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt)
        part[rr][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(f16x8, t.b[tt][s]),
                                                               part[rr][tt], 0, 0, 0);
    }
  }
  // the tile's sums times the token's 2^-p (exact) into the accumulator; D column = token = lane % 16
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) {
      const float u = __uint_as_float(t.xu[tt]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[rr][tt][e] = __builtin_fmaf(part[rr][tt][e], u, acc[rr][tt][e]);
    }
}

// LoRA-up operands of one row-group slot: rows of B (bf16, ranks past r read as 0) and the t fragments.
template <int TMT>
struct LoraOps {
  u32x4 bfrag[kRankChunks];
  u32x4 thi[kRankChunks][TMT], tlo[kRankChunks][TMT];
};

// LoRA-up operands in two steps: issue (rows of B and the raw k-chunk partials of t, before the weight stream) and
// finish (after it: partials summed in chunk order, split into bf16 hi and lo parts).
template <int TMT>
struct LoraRaw {
  u32x4 part[kRankChunks][TMT][2];  // the first k-chunk's partial (the whole t when k <= 4096)
};

template <int TMT>
__device__ __forceinline__ void issue_lora(LoraOps<TMT>& o, LoraRaw<TMT>& raw, const ProjArgs& P, int p, int64_t rg,
                                           int lane, const LinearArgs& a, int64_t tile0, int64_t ntiles) {
  const int64_t n = rg * 16 + lane % 16;
  const rsrc_t bsrc = make_rsrc(P.B, P.n * P.r * 2), tsrc = make_rsrc(a.t_part, a.t_bytes);
#pragma unroll
  for (int jc = 0; jc < kRankChunks; ++jc) {
    const int j0 = jc * 32 + (lane / 16) * 8;
    if (P.r % 8 == 0) {
      o.bfrag[jc] = bload16(bsrc, (n < P.n && j0 < P.r) ? (uint32_t)((n * P.r + j0) * 2) : kOutOfRange);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t off = (n * P.r + j0 + 2 * e) * 2;
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
            bsrc, (n < P.n && j0 + 2 * e < P.r) ? (uint32_t)off : kOutOfRange, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
            bsrc, (n < P.n && j0 + 2 * e + 1 < P.r) ? (uint32_t)(off + 2) : kOutOfRange, 0, 0);
        w[e] = lo | (hi << 16);
      }
      o.bfrag[jc] = u32x4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) {
      const bool ok = jc * 32 < P.r && tile0 + tt < ntiles;
      const uint32_t off =
          (uint32_t)((((((int64_t)p * ntiles + tile0 + tt) * kRankChunks + jc) * a.ks) * kWave + lane) * 32);
      raw.part[jc][tt][0] = bload16(tsrc, ok ? off : kOutOfRange);
      raw.part[jc][tt][1] = bload16(tsrc, ok ? off + 16 : kOutOfRange);
    }
  }
}

template <int TMT>
__device__ __forceinline__ void finish_lora(LoraOps<TMT>& o, const LoraRaw<TMT>& raw, const ProjArgs& P, int p,
                                            int lane, const LinearArgs& a, int64_t tile0, int64_t ntiles) {
#pragma unroll
  for (int jc = 0; jc < kRankChunks; ++jc)
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) {
      f32x4 s0 = __builtin_bit_cast(f32x4, raw.part[jc][tt][0]);
      f32x4 s1 = __builtin_bit_cast(f32x4, raw.part[jc][tt][1]);
      const bool ok = jc * 32 < P.r && tile0 + tt < ntiles;
      const rsrc_t tsrc = make_rsrc(a.t_part, a.t_bytes);
      const uint32_t off =
          (uint32_t)((((((int64_t)p * ntiles + tile0 + tt) * kRankChunks + jc) * a.ks) * kWave + lane) * 32);
      // the remaining chunks, in chunk order; loads issued eight chunks at a time
      for (int c0 = 1; c0 < a.ks; c0 += 8) {
        u32x4 q[8][2];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t oc = off + (uint32_t)(c0 + u) * kWave * 32;
          const bool in = ok && c0 + u < a.ks;
          q[u][0] = bload16(tsrc, in ? oc : kOutOfRange);
          q[u][1] = bload16(tsrc, in ? oc + 16 : kOutOfRange);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {  // loads past the last chunk read 0 and add nothing
          s0 += __builtin_bit_cast(f32x4, q[u][0]);
          s1 += __builtin_bit_cast(f32x4, q[u][1]);
        }
      }
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = e < 4 ? s0[e] : s1[e - 4];
        const uint32_t th = f32_to_bf16(t);
        const uint32_t tl = f32_to_bf16(t - bf16_to_f32((uint16_t)th));  // t - th is exact in f32
        if (e % 2 == 0) {
          hi[e / 2] = th;
          lo[e / 2] = tl;
        } else {
          hi[e / 2] |= th << 16;
          lo[e / 2] |= tl << 16;
        }
      }
      o.thi[jc][tt] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      o.tlo[jc][tt] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
}

template <int TMT>
__device__ __forceinline__ void lora_mfma(const LoraOps<TMT>& o, f32x4 (&acc)[TMT]) {
#pragma unroll
  for (int jc = 0; jc < kRankChunks; ++jc)
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) {
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, o.bfrag[jc]),
                                                        __builtin_bit_cast(bf16x8, o.thi[jc][tt]), acc[tt], 0, 0, 0);
      acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, o.bfrag[jc]),
                                                        __builtin_bit_cast(bf16x8, o.tlo[jc][tt]), acc[tt], 0, 0, 0);
    }
}

// What the epilogue needs of the projection an output slot belongs to (n = 0 for a slot past the last row group).
struct SlotOut {
  void* y;
  const uint16_t* res;
  int64_t n, ldy, ld_res, n0;  // n0: first output row of the slot
  int32_t y_dtype, y_repeat, head_dim;
};

template <int TMT, int R, int W, bool SILU>
__global__ void __launch_bounds__(W * kWave) k_linear(LinearArgs a) {
  constexpr int kSlots = SILU ? R / 2 : R;                  // output row groups per workgroup
  constexpr int kOut = (kSlots * 16 * TMT * 16 + W * kWave - 1) / (W * kWave);  // outputs per thread (max)
  constexpr bool kEarlyLora = TMT <= 2;                     // LoRA operands fetched before the weight stream
  __shared__ f32x4 red[W + 1][R][TMT][kWave];               // wave partials; [W] holds the LoRA-up products
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int64_t KT = a.kp / kKTile;

  // row group of every slot
  int pj[R];
  int64_t rg[R];
  bool live[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (SILU) {
      pj[rr] = rr % 2;
      rg[rr] = (int64_t)blockIdx.x * (R / 2) + rr / 2;
      live[rr] = rg[rr] * 16 < a.p[0].n;
    } else {
      const int64_t g = (int64_t)blockIdx.x * R + rr;
      int p = 0;
      while (p + 1 < a.nproj && g >= a.p[p + 1].rg_begin) ++p;
      pj[rr] = p;
      rg[rr] = g - a.p[p].rg_begin;
      live[rr] = rg[rr] * 16 < a.p[p].n;
    }
  }
  const int64_t mrem = a.m - a.tok0;
  const int mt = (int)(mrem < TMT * 16 ? mrem : TMT * 16);  // tokens in this launch
  const int64_t tile0 = a.tok0 / 16, ntiles = ceil_div(a.m, 16);

  // Per-slot epilogue constants, read once (wave-uniform) and selected per output from registers: indexing the
  // argument block with a per-lane slot would turn each read into a dependent vector load.
  constexpr int kPer = SILU ? 2 : 1;
  SlotOut so[kSlots];
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl) {
    const ProjArgs& P = a.p[pj[sl * kPer]];
    so[sl] = SlotOut{P.y, P.res, live[sl * kPer] ? P.n : 0, P.ldy, P.ld_res, rg[sl * kPer] * 16, P.y_dtype,
                     P.y_repeat, P.head_dim};
  }
  float sgv[R], lam[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    sgv[rr] = gload(a.p[pj[rr]].s_g);
    lam[rr] = a.p[pj[rr]].lambda;
  }

  // epilogue operand fetched now, consumed after the weight stream: per output the residual (an unconditional load:
  // outputs the epilogue skips read a valid stand-in address instead)
  uint16_t res[kOut];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int o = threadIdx.x + i * W * kWave;
    const int row = o % 16, tok = (o / 16) % mt, slot = o / (16 * mt);
    const uint16_t* rp = reinterpret_cast<const uint16_t*>(a.xsc);
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
      const int64_t n = so[sl].n0 + row;
      if (slot == sl && so[sl].res && n < so[sl].n) rp = so[sl].res + (a.tok0 + tok) * so[sl].ld_res + n;
    }
    res[i] = gload(rp);
  }
  // LoRA-up: wave w owns the slots rr with rr % W == w (lops / lraw index rr / W)
  constexpr int kLoraSlots = (R + W - 1) / W;
  LoraOps<TMT> lops[kLoraSlots];
  LoraRaw<TMT> lraw[kLoraSlots];
  if (kEarlyLora) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
      if (rr % W == wave && a.p[pj[rr]].r > 0)
        issue_lora<TMT>(lops[rr / W], lraw[rr / W], a.p[pj[rr]], pj[rr], rg[rr], lane, a, tile0, ntiles);
  }

  Streams<TMT, R> st;
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const ProjArgs& P = a.p[pj[rr]];
    st.c[rr] = make_rsrc(P.codes + rg[rr] * KT * kTileCodeBytes, live[rr] ? KT * kTileCodeBytes : 0);
    st.s[rr] = make_rsrc(P.scales + rg[rr] * KT * kTileScaleBytes, live[rr] ? KT * kTileScaleBytes : 0);
  }
  st.c_off = lane * 16;
  st.s_off = ((lane % 16) * 2 + (lane / 16) / 2) * 4;
  st.b = make_rsrc(a.xs + tile0 * KT * 4 * kWave, TMT * KT * 4 * kWave * 16);
  st.x = make_rsrc(a.xsc + tile0 * KT * 16, TMT * KT * 16 * 4);
#pragma unroll
  for (int tt = 0; tt < TMT; ++tt) {
    const bool in = tt * 16 + lane % 16 < mt;
    st.b_off[tt] = in ? (uint32_t)((tt * KT * 4 * kWave + lane) * 16) : kOutOfRange;
    st.x_off[tt] = in ? (uint32_t)((tt * KT * 16 + lane % 16) * 4) : kOutOfRange;
  }

  f32x4 acc[R][TMT];
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) acc[rr][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two tile buffers: the loads of the next tile (index clamped to the wave's last tile, so they are unconditional
  // and the compiler's wait counts stay exact) are in flight while the current tile is converted and multiplied.
  const int64_t kb = wave * KT / W, ke = (wave + 1) * KT / W;
  if (kb < ke) {
    TileBuf<TMT, R> t0, t1;
    load_tile<TMT, R>(t0, st, kb);
    for (int64_t kt = kb; kt < ke; kt += 2) {
      load_tile<TMT, R>(t1, st, kt + 1 < ke ? kt + 1 : ke - 1);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute it overlaps
      compute_tile<TMT, R>(t0, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 >= ke) break;
      load_tile<TMT, R>(t0, st, kt + 2 < ke ? kt + 2 : ke - 1);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile<TMT, R>(t1, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) red[wave][rr][tt][lane] = acc[rr][tt];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (rr % W != wave) continue;
    const int q = rr / W;
    f32x4 la[TMT];
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) la[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.p[pj[rr]].r > 0) {
      if (!kEarlyLora) issue_lora<TMT>(lops[q], lraw[q], a.p[pj[rr]], pj[rr], rg[rr], lane, a, tile0, ntiles);
      finish_lora<TMT>(lops[q], lraw[q], a.p[pj[rr]], pj[rr], lane, a, tile0, ntiles);
      lora_mfma<TMT>(lops[q], la);
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt) mfma_settle(la[tt]);  // (read past the end of this branch)
    }
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) red[W][rr][tt][lane] = la[tt];
  }
  __syncthreads();

  // Epilogue: one output (slot, row, token) per thread step; rows vary fastest so stores are contiguous.
  const int nout = kSlots * 16 * mt;
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int o = threadIdx.x + i * W * kWave;
    if (o >= nout) break;
    const int row = o % 16;
    const int tok = (o / 16) % mt;
    const int slot = o / (16 * mt);
    const int tt = tok / 16, col = tok % 16;
    const int ln = (row / 4) * 16 + col, ii = row % 4;
    const int64_t gtok = a.tok0 + tok;
    float val[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int rr = slot * kPer + q;
      float sg = sgv[q], lm = lam[q];
#pragma unroll
      for (int r2 = kPer + q; r2 < R; r2 += kPer)
        if (rr == r2) {
          sg = sgv[r2];
          lm = lam[r2];
        }
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) s += red[w][rr][tt][ln][ii];
      val[q] = sg * s + lm * red[W][rr][tt][ln][ii];
    }
    SlotOut O = so[0];
#pragma unroll
    for (int sl = 1; sl < kSlots; ++sl)
      if (slot == sl) O = so[sl];
    const int64_t n = O.n0 + row;
    if (n >= O.n) continue;
    float out = val[0];
    if (SILU) {
      const float g = val[0];
      out = g / (1.0f + __expf(-g)) * val[kPer - 1];
    }
    if (O.res) out += bf16_to_f32(res[i]);
    store_output(O.y, O.y_dtype, gtok * O.ldy, n, O.y_repeat, O.head_dim, out);
  }
}

// ------------------------------------------------------------------------------------------------------------------
// G: decode streaming kernel for up to 32 tokens per launch (TMT = 1 or 2 token tiles of 16).
//   Work is row units (a row group of 16 rows; with SILU a (gate, up) pair of row groups) x k-tiles, cut into
//   nbr row blocks x nk k-chunks, one workgroup each; the host sizes the cut so the grid is about one workgroup per CU
//   with equal shares. The workgroup copies the activation fragments and tile scales of its k-chunk into LDS once;
//   waves 0..14 split the block's units (and, with fewer units than waves, the chunk's k-tiles between them) and load
//   only weights from memory, D tiles in flight each; wave 15 computes the LoRA-up term B t of the block's rows
//   meanwhile (in the chunk-0 workgroup). With nk > 1 every workgroup stores its part sums, and the last of a block's
//   workgroups to arrive (an atomic counter) adds the nk parts in chunk order and runs the epilogue, so results do not
//   depend on scheduling.
constexpr int kGWaves = 16;
constexpr int kGStream = kGWaves - 1;
constexpr int kGMaxUnits = 8;
constexpr int kGLds = 144 * 1024;                   // LDS bytes per workgroup (besides the residual tile)
constexpr int kGTileAct = 4 * kWave * 16 + 16 * 4;  // LDS bytes per (k-tile, token tile): 4 fragments + 16 scales
constexpr int kGFragLoads = 10;                     // 16-byte activation loads per thread (at most)
__host__ __device__ constexpr int gemv_lred_bytes(int nr, int tmt) { return kGMaxUnits * nr * tmt * kWave * 16; }
__host__ __device__ constexpr int64_t gemv_block_floats(int nr, int tmt) { return (int64_t)kGMaxUnits * nr * tmt * 256; }

__host__ __device__ constexpr int vmcnt_imm(int n) {  // s_waitcnt immediate: vmcnt = n, expcnt and lgkmcnt not waited
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

struct GemvArgs {
  LinearArgs L;
  int32_t nu, nbr, nk;
  int32_t KT, ntiles, mt;  // k-tiles, token tiles, tokens (32-bit copies: the kernel's preamble avoids 64-bit division)
  float* pbuf;    // [nbr][nk + 1][gemv_block_floats] part sums; slot nk holds the LoRA term
  uint32_t* cnt;  // [nbr] arrival counters, zero between calls
};

// Per-projection epilogue data, staged in LDS so that each output reads its projection's entry by index.
struct ProjEpi {
  void* y;
  const uint16_t* res;
  int64_t n, ldy, ld_res;
  float sg, lambda;
  int32_t y_dtype, y_repeat, head_dim, rg_begin, r;
};

template <int NR>
struct GTile {
  u32x4 c[NR];
  uint32_t sc[NR];
};

// Projection and row group of row unit g (flattened over the projections; with SILU both projections' group g).
__device__ __forceinline__ int unit_proj(const ProjEpi* pe, int nproj, int64_t g) {
  int p = 0;
  for (int q = 1; q < nproj; ++q)
    if (g >= pe[q].rg_begin) p = q;
  return p;
}

// Split-k reduction and epilogue of the decode kernels. Thread t of the NTHR holds the sums (vsum) and LoRA terms
// (vlo, valid in chunk 0) of outputs e = t + i * NTHR, i < KOUT, e = (unit * TMT*16 + token) * 16 + row, e < nout.
// With a split k, every chunk stores its sums and the last workgroup of the row block to arrive adds them in chunk
// order; the others return. The sums are written and read with device-scope relaxed atomic accesses, which go to
// memory past the per-XCD L2 caches; the stores have completed (s_waitcnt) before the workgroup's barrier and its
// arrival, so no cache-wide fence is needed (no L2 writeback or invalidation). Then y = s_g * sum + lambda * lora
// (SILU: SiLU(gate) * up), + residual (s_res, in output order), broadcast and rounding.
template <int TMT, bool SILU, int KOUT, int NTHR>
__device__ __forceinline__ void gemv_finish(const GemvArgs& g, const ProjEpi* s_pe, const uint16_t* s_res, int* s_last,
                                            float (&vsum)[KOUT][SILU ? 2 : 1], float (&vlo)[KOUT][SILU ? 2 : 1],
                                            int nout, int b, int c, int u0) {
  constexpr int NR = SILU ? 2 : 1;
  constexpr int kOut = KOUT;
  const LinearArgs& a = g.L;
  const int mt = g.mt;
  if (g.nk > 1) {
    const int64_t PB = gemv_block_floats(NR, TMT);
    float* pb = g.pbuf + (int64_t)b * (g.nk + 1) * PB;
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int e = threadIdx.x + i * NTHR;
      if (e >= nout) break;
#pragma unroll
      for (int nr = 0; nr < NR; ++nr) {
        __hip_atomic_store(pb + (int64_t)c * PB + (int64_t)e * NR + nr, vsum[i][nr], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (c == 0)
          __hip_atomic_store(pb + (int64_t)g.nk * PB + (int64_t)e * NR + nr, vlo[i][nr], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // every store of this thread has completed
    __syncthreads();
    if (threadIdx.x == 0)
      *s_last = __hip_atomic_fetch_add(g.cnt + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (uint32_t)(g.nk - 1);
    __syncthreads();
    if (!*s_last) return;
    // every output's chunk sums, kRedBatch chunks per batch of loads issued together (one memory round trip per
    // batch, where one load after another would cost a round trip each), added in chunk order
    constexpr int kRedBatch = 8;
#pragma unroll
    for (int i = 0; i < kOut; ++i)
#pragma unroll
      for (int nr = 0; nr < NR; ++nr) vsum[i][nr] = 0.f;
    for (int c0 = 0; c0 < g.nk; c0 += kRedBatch) {
      float q[kOut][NR][kRedBatch];
#pragma unroll
      for (int i = 0; i < kOut; ++i) {
        const int e = threadIdx.x + i * NTHR;
#pragma unroll
        for (int nr = 0; nr < NR; ++nr)
#pragma unroll
          for (int v = 0; v < kRedBatch; ++v)
            q[i][nr][v] = (e < nout && c0 + v < g.nk)
                              ? __hip_atomic_load(pb + (int64_t)(c0 + v) * PB + (int64_t)e * NR + nr, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                              : 0.f;
        if (c0 == 0) {
#pragma unroll
          for (int nr = 0; nr < NR; ++nr)
            vlo[i][nr] = e < nout ? __hip_atomic_load(pb + (int64_t)g.nk * PB + (int64_t)e * NR + nr,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                  : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < kOut; ++i)
#pragma unroll
        for (int nr = 0; nr < NR; ++nr)
#pragma unroll
          for (int v = 0; v < kRedBatch; ++v) {
            if (c0 + v >= g.nk) break;
            vsum[i][nr] = (c0 + v == 0) ? q[i][nr][v] : vsum[i][nr] + q[i][nr][v];
          }
    }
    if (threadIdx.x == 0) __hip_atomic_store(g.cnt + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 6. epilogue: y = s_g * sum + lambda * lora (SILU: SiLU(gate) * up), + residual, broadcast, rounding
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int e = threadIdx.x + i * NTHR;
    if (e >= nout) break;
    const int u = (int)((unsigned)e / (TMT * 256)), tok = (e >> 4) & (TMT * 16 - 1), row = e & 15;
    if (tok >= mt) continue;
    const int64_t gu = u0 + u;
    const int p0 = SILU ? 0 : unit_proj(s_pe, a.nproj, gu);
    const ProjEpi& E = s_pe[p0];
    const int64_t n = (SILU ? gu : gu - E.rg_begin) * 16 + row;
    if (n >= E.n) continue;
    float val[NR];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      const ProjEpi& F = s_pe[SILU ? nr : p0];
      val[nr] = F.sg * vsum[i][nr] + F.lambda * vlo[i][nr];
    }
    float out = val[0];
    if (SILU) out = val[0] / (1.0f + __expf(-val[0])) * val[NR - 1];
    if (E.res) out += bf16_to_f32(s_res[e]);
    const int64_t gtok = a.tok0 + tok;
    store_output(E.y, E.y_dtype, gtok * E.ldy, n, E.y_repeat, E.head_dim, out);
  }
}

template <int TMT, bool SILU, int D>
__global__ void __launch_bounds__(kGWaves * kWave) k_gemv(GemvArgs g) {
  constexpr int NR = SILU ? 2 : 1;
  constexpr int kOut = (kGMaxUnits * 16 * TMT * 16 + kGWaves * kWave - 1) / (kGWaves * kWave);
  constexpr int kTBatch = 4 / TMT;  // LoRA-down chunk partials loaded together
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kGLds];
  __shared__ uint16_t s_res[kGMaxUnits * 16 * TMT * 16];  // residual of each output (epilogue order)
  __shared__ ProjEpi s_pe[kMaxProj];
  __shared__ int s_last;
  const LinearArgs& a = g.L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const unsigned bid = blockIdx.x, nbr = (unsigned)g.nbr, nk = (unsigned)g.nk;
  const int b = (int)(bid % nbr), c = (int)(bid / nbr);
  const int KT = g.KT, mt = g.mt, ntiles = g.ntiles;
  const int u0 = (int)((unsigned)b * (unsigned)g.nu / nbr);
  const int U = (int)((unsigned)(b + 1) * (unsigned)g.nu / nbr) - u0;
  const int t0 = (int)((unsigned)c * (unsigned)KT / nk), T = (int)((unsigned)(c + 1) * (unsigned)KT / nk) - t0;
  constexpr int64_t tile0 = 0;  // one launch covers every token (at most 32)
  const int ntl = ntiles < TMT ? ntiles : TMT;  // token tiles present
  uint8_t* const lred = s_lds + kGLds - gemv_lred_bytes(NR, TMT);
  const int fr_bytes = TMT * T * 4 * kWave * 16;

  // 1. stream waves: unit u, k-part j of h. The preamble is kept short because every instruction of it is fetched
  //    cold at each launch.
  constexpr unsigned char kParts[kGMaxUnits + 1] = {1, 15, 7, 5, 3, 3, 2, 2, 1};  // kGStream / U
  static_assert(kGStream == 15 && kGMaxUnits == 8, "parts table");
  const int h = kParts[U];
  const bool streams = wave < U * h;
  const int su = streams ? (int)((unsigned)wave / (unsigned)h) : 0, sj = streams ? wave - su * h : 0;
  // wave-uniform tile range (readfirstlane: keeps the loop counter scalar and the loop's wait counts exact)
  const int ta = __builtin_amdgcn_readfirstlane(t0 + (int)((unsigned)(sj * T) / (unsigned)h));
  const int tb = __builtin_amdgcn_readfirstlane(streams ? t0 + (int)((unsigned)((sj + 1) * T) / (unsigned)h) : ta);
  rsrc_t cd[NR], sd[NR];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    const int64_t gu = u0 + su;
    int p = nr;
    if (!SILU) {
      p = 0;
      for (int q = 1; q < a.nproj; ++q)
        if (gu >= a.p[q].rg_begin) p = q;
      p = __builtin_amdgcn_readfirstlane(p);
    }
    const ProjArgs& P = a.p[p];
    const int64_t rg = SILU ? gu : gu - P.rg_begin;
    const bool live = streams && rg * 16 < P.n;
    cd[nr] = make_rsrc(P.codes + rg * KT * kTileCodeBytes, live ? KT * kTileCodeBytes : 0);
    sd[nr] = make_rsrc(P.scales + rg * KT * kTileScaleBytes, live ? KT * kTileScaleBytes : 0);
  }
  const uint32_t c_off = lane * 16, s_off = ((lane % 16) * 2 + (lane / 16) / 2) * 4;
  auto load = [&](GTile<NR>& t, int kt) {
    const bool in = kt < tb;
    const int kc = __builtin_amdgcn_readfirstlane(in ? kt * kTileCodeBytes : 0);
    const int ks = __builtin_amdgcn_readfirstlane(in ? kt * kTileScaleBytes : 0);
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      t.c[nr] = __builtin_amdgcn_raw_buffer_load_b128(cd[nr], in ? c_off : kOutOfRange, kc, kNonTemporal);
      t.sc[nr] = __builtin_amdgcn_raw_buffer_load_b32(sd[nr], in ? s_off : kOutOfRange, ks, kNonTemporal);
    }
  };
  GTile<NR> Bt[D];

  // 2. the chunk's activation fragments ([tt][lt][s][lane], 16 bytes) and tile scales ([tt][lt][16] f32), loaded
  //    straight into LDS (1 KB per wave and step; a chunk never straddles token tiles: T * 256 is a multiple of 64)
  const int nfc = TMT * T * 4 * kWave, nsc = TMT * T * 4;  // 16-byte pieces of fragments, of scales
  {
    const rsrc_t xsrc = make_rsrc(a.xs + tile0 * KT * 4 * kWave, (int64_t)ntl * KT * 4 * kWave * 16);
    for (int ch = wave; ch * kWave < nfc; ch += kGWaves) {
      const int q0 = ch * kWave, tt = q0 >= T * 4 * kWave ? 1 : 0, rem = q0 - tt * T * 4 * kWave;  // TMT <= 2
      const int so = __builtin_amdgcn_readfirstlane((int)((((int64_t)tt * KT + t0) * 4 * kWave + rem) * 16));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrc, (__attribute__((address_space(3))) void*)(s_lds + q0 * 16), 16,
                                               lane * 16, so, 0, 0);
    }
    const rsrc_t ssrc = make_rsrc(a.xsc + tile0 * KT * 16, (int64_t)ntl * KT * 16 * 4);
    for (int ch = wave; ch * kWave < nsc; ch += kGWaves) {
      // scale piece q: token tile q / (T*4), then 16 bytes of the [lt][16] block; lanes past nsc load nothing
      const int q = ch * kWave + lane, tt = q >= T * 4 ? 1 : 0, rem = q - tt * T * 4;  // TMT <= 2
      if (q < nsc)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ssrc, (__attribute__((address_space(3))) void*)(s_lds + fr_bytes + ch * kWave * 16), 16,
            (uint32_t)((((int64_t)tt * KT + t0) * 16) * 4 + rem * 16), 0, 0, 0);
    }
  }
  if (threadIdx.x < kMaxProj) {
#pragma unroll
    for (int q = 0; q < kMaxProj; ++q)
      if (threadIdx.x == q && q < a.nproj) {
        const ProjArgs& P = a.p[q];
        s_pe[q] = ProjEpi{P.y, P.res, P.n, P.ldy, P.ld_res, gload(P.s_g), P.lambda, P.y_dtype, P.y_repeat,
                          P.head_dim, P.rg_begin, P.r};
      }
  }
  // residual of this thread's outputs (output e = (unit, token, row) = ((u * TMT*16 + tok) * 16 + row)); outputs
  // without one read a valid stand-in address. Issued here, the barrier's wait covers them at no extra cost.
  uint16_t res[kOut];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int e = threadIdx.x + i * kGWaves * kWave;
    const int u = e >> (TMT == 1 ? 8 : 9), tok = (e >> 4) & (TMT * 16 - 1), row = e & 15;
    const int64_t gu = u0 + u;
    const uint16_t* rb = a.p[0].res;
    int64_t rbeg = 0, nl = a.p[0].n, ld = a.p[0].ld_res;
    if (!SILU) {
#pragma unroll
      for (int q = 1; q < kMaxProj; ++q)
        if (q < a.nproj && gu >= a.p[q].rg_begin) {
          rb = a.p[q].res;
          rbeg = a.p[q].rg_begin;
          nl = a.p[q].n;
          ld = a.p[q].ld_res;
        }
    }
    const int64_t n = (gu - rbeg) * 16 + row;
    const bool ok = rb && u < U && tok < mt && n < nl;
    res[i] = gload(ok ? rb + tok * ld + n : reinterpret_cast<const uint16_t*>(a.xsc));
  }
  // the first D - 1 weight tiles (from HBM) are requested after the activation copies and residuals: loads return
  // in order, so the wait below covers those (loads to LDS are counted by vmcnt) and not these tiles, which stay in
  // flight across the barrier (requested first, they held up every wave's copy: measured 0.6-0.8 us slower)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < D - 1; ++j) {
    load(Bt[j], ta + j);
    __builtin_amdgcn_sched_barrier(0);  // issue order of the first tiles: the loop's wait counts rely on it
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 1) * NR * 2));
#pragma unroll
  for (int i = 0; i < kOut; ++i) s_res[threadIdx.x + i * kGWaves * kWave] = res[i];
  __syncthreads();

  f32x4 acc[NR][TMT];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr)
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) acc[nr][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // (a tile past the wave's range has zero weights; its activations are read at the last tile of the range, which
  // are finite, so it adds exactly zero)
  auto compute = [&](const GTile<NR>& t, int kt) {
    const int lt = (kt < tb ? kt : tb - 1) - t0;
    f32x4 part[NR][TMT];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt) part[nr][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 bf[TMT];
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt)
        bf[tt] = *reinterpret_cast<const u32x4*>(s_lds + (((tt * T + lt) * 4 + s) * kWave + lane) * 16);
#pragma unroll
      for (int nr = 0; nr < NR; ++nr) {
        const uint32_t scv = ((t.sc[nr] >> (8 * s)) & 0xFFu) * 0x00800080u;  // E4M3 byte << 7 = E4M3 * 2^-8 in f16
        const f16x2 sh = __builtin_bit_cast(f16x2, scv);
        const uint32_t cw = t.c[nr][s];
        const f16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 0) * sh;
        const f16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 1) * sh;
        const f16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 2) * sh;
        const f16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 3) * sh;
        const f16x8 wv = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
#pragma unroll
        for (int tt = 0; tt < TMT; ++tt)
          part[nr][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, __builtin_bit_cast(f16x8, bf[tt]), part[nr][tt],
                                                                0, 0, 0);
      }
    }
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) {
      const float u = *reinterpret_cast<const float*>(s_lds + fr_bytes + ((tt * T + lt) * 16 + lane % 16) * 4);
#pragma unroll
      for (int nr = 0; nr < NR; ++nr)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[nr][tt][e] = __builtin_fmaf(part[nr][tt][e], u, acc[nr][tt][e]);
    }
  };

  if (streams) {
    // D tiles in flight: the load D - 1 tiles ahead is issued before the current tile is computed (D = 3 measured
    // best; deeper prefetch was slower at the 7B shapes). The body has no early exit (a loop with several exits gets
    // flow edges that make the compiler's wait counts conservative); tiles past the range are loaded out of range (no
    // memory traffic) and add zero.
    for (int kt = ta; kt < tb; kt += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        load(Bt[(j + D - 1) % D], kt + j + D - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(Bt[j], kt + j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // (a separate block after the loop, so that the loop's entry state holds the stream's loads only)
  if (wave == kGWaves - 1 && c == 0) {
    // 3. LoRA-up of the block's rows: per projection and 32-rank chunk, t (the LoRA-down chunk partials summed in
    //    chunk order, split into bf16 hi and lo parts), then two bf16 MFMAs per unit, accumulated over rank chunks
    //    in LDS. Lane layouts: B rows (lane%16 = row, ranks 8 (lane/16) ..) and t (lane%16 = token, same ranks).
    //    The rows of B of every unit are requested before the chunk partials of t, so a rank chunk costs as many
    //    memory round trips as there are batches of partials, while the weights stream.
    const rsrc_t tsrc = make_rsrc(a.t_part, a.t_bytes);
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      int pfirst = SILU ? nr : unit_proj(s_pe, a.nproj, u0), plast = SILU ? nr : unit_proj(s_pe, a.nproj, u0 + U - 1);
      pfirst = __builtin_amdgcn_readfirstlane(pfirst);
      plast = __builtin_amdgcn_readfirstlane(plast);
      for (int p = pfirst; p <= plast; ++p) {
        const ProjEpi& E = s_pe[p];
        const uint16_t* Bm = nullptr;
#pragma unroll
        for (int q = 0; q < kMaxProj; ++q)
          if (q == p) Bm = a.p[q].B;
        const int r = E.r;
        for (int jc = 0; jc * 32 < r; ++jc) {
          const rsrc_t bsrc = make_rsrc(Bm, E.n * r * 2);
          // rows of B for every unit of the block that belongs to projection p (others read 0)
          u32x4 bfr[kGMaxUnits];
#pragma unroll
          for (int u = 0; u < kGMaxUnits; ++u) {
            const bool mine = u < U && (SILU || unit_proj(s_pe, a.nproj, u0 + u) == p);
            const int64_t n = (SILU ? u0 + u : u0 + u - E.rg_begin) * 16 + lane % 16;
            const int j0 = jc * 32 + (lane / 16) * 8;
            if (r % 8 == 0) {
              bfr[u] = bload16(bsrc, (mine && n < E.n && j0 < r) ? (uint32_t)((n * r + j0) * 2) : kOutOfRange);
            } else {
              uint32_t w[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int64_t off = (n * r + j0 + 2 * e) * 2;
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                    bsrc, (mine && n < E.n && j0 + 2 * e < r) ? (uint32_t)off : kOutOfRange, 0, 0);
                const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                    bsrc, (mine && n < E.n && j0 + 2 * e + 1 < r) ? (uint32_t)(off + 2) : kOutOfRange, 0, 0);
                w[e] = lo | (hi << 16);
              }
              bfr[u] = u32x4{w[0], w[1], w[2], w[3]};
            }
          }
          // per token tile: t (chunk partials in chunk order, kTBatch chunks per batch of loads; loads past the
          // last chunk read 0 and add nothing), then B t for the units of this projection, added into the LDS slot
          // (unit, nr, tt)
#pragma unroll
          for (int tt = 0; tt < TMT; ++tt) {
            const bool ok = tt < ntl;
            const uint32_t off =
                (uint32_t)((((((int64_t)p * ntiles + tile0 + tt) * kRankChunks + jc) * a.ks) * kWave + lane) * 32);
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            for (int c0 = 0; c0 < a.ks; c0 += kTBatch) {
              u32x4 q[kTBatch][2];
#pragma unroll
              for (int v = 0; v < kTBatch; ++v) {
                const bool in = ok && c0 + v < a.ks;
                const uint32_t oc = off + (uint32_t)(c0 + v) * kWave * 32;
                q[v][0] = bload16(tsrc, in ? oc : kOutOfRange);
                q[v][1] = bload16(tsrc, in ? oc + 16 : kOutOfRange);
              }
#pragma unroll
              for (int v = 0; v < kTBatch; ++v) {
                s0 += __builtin_bit_cast(f32x4, q[v][0]);
                s1 += __builtin_bit_cast(f32x4, q[v][1]);
              }
            }
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float t = e < 4 ? s0[e] : s1[e - 4];
              const uint32_t th = f32_to_bf16(t);
              const uint32_t tl = f32_to_bf16(t - bf16_to_f32((uint16_t)th));  // t - th is exact in f32
              if (e % 2 == 0) {
                hi[e / 2] = th;
                lo[e / 2] = tl;
              } else {
                hi[e / 2] |= th << 16;
                lo[e / 2] |= tl << 16;
              }
            }
            const u32x4 thi = u32x4{hi[0], hi[1], hi[2], hi[3]}, tlo = u32x4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
            for (int u = 0; u < kGMaxUnits; ++u) {
              if (u >= U) break;
              if (!SILU && unit_proj(s_pe, a.nproj, u0 + u) != p) continue;
              f32x4 la = {0.f, 0.f, 0.f, 0.f};
              la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr[u]),
                                                           __builtin_bit_cast(bf16x8, thi), la, 0, 0, 0);
              la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr[u]),
                                                           __builtin_bit_cast(bf16x8, tlo), la, 0, 0, 0);
              mfma_settle(la);  // (the store below sits behind a branch on one of its paths)
              f32x4* slot = reinterpret_cast<f32x4*>(lred + ((((u * NR + nr) * TMT + tt) * kWave) + lane) * 16);
              *slot = jc == 0 ? la : *slot + la;
            }
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done with the activations in LDS

  // 4. part sums of the stream waves into LDS (over the activation area), then the per-output sums
  if (streams) {
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt)
        *reinterpret_cast<f32x4*>(s_lds + (((((su * h + sj) * NR + nr) * TMT + tt) * kWave) + lane) * 16) =
            acc[nr][tt];
  }
  __syncthreads();

  const bool has_lora = c == 0;  // LoRA slots were written in chunk 0 (zero where the projection has no adapter)
  const int nout = U * TMT * 256;  // outputs (unit, token, row); tokens past mt are skipped
  float vsum[kOut][NR], vlo[kOut][NR];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int e = threadIdx.x + i * kGWaves * kWave;
    const int u = e >> (TMT == 1 ? 8 : 9), tok = (e >> 4) & (TMT * 16 - 1), row = e & 15;
    const int tt = tok / 16, col = tok % 16;
    const int ln = (row / 4) * 16 + col, ii = row % 4;
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      float s = 0.f, lo = 0.f;
      if (e < nout) {
        for (int j = 0; j < h; ++j)
          s += reinterpret_cast<const float*>(s_lds + (((((u * h + j) * NR + nr) * TMT + tt) * kWave) + ln) * 16)[ii];
        if (has_lora && s_pe[SILU ? nr : unit_proj(s_pe, a.nproj, u0 + u)].r > 0)
          lo = reinterpret_cast<const float*>(lred + ((((u * NR + nr) * TMT + tt) * kWave) + ln) * 16)[ii];
      }
      vsum[i][nr] = s;
      vlo[i][nr] = lo;
    }
  }

  gemv_finish<TMT, SILU, kOut, kGWaves * kWave>(g, s_pe, s_res, &s_last, vsum, vlo, nout, b, c, u0);
}

// ------------------------------------------------------------------------------------------------------------------
// W: decode kernel for 17 to 64 tokens (TMT = 2 or 4 token tiles). At these token counts the activations of a whole
// k-chunk no longer fit in LDS beside the rows' work, so they stream through it. A chunk's k-tiles are taken in passes
// of kWH; a pass's activation fragments and tile scales are loaded straight into one of NB LDS buffers, LA = NB - 1
// passes ahead, while the waves compute the current pass from another. Stream wave w serves unit slot w / kWH and
// the k-tile w % kWH of every pass, so all stream waves move through k together and every activation tile in LDS
// feeds all units of the workgroup: activations are read once per workgroup, weights once. Each wave keeps its own
// weight tiles LW passes ahead in registers. One barrier per pass (after each wave's own loads into the pass's
// buffer have landed) publishes the buffer and frees the one filled next. Every buffer is an LDS array of its own,
// so the compiler sees that the fills in flight never overlap the buffer being read and adds no wait for them.
// Wave 15 computes the LoRA-up of the block's units from the finished LoRA-down t (bf16 hi and lo fragments) and the
// rows of B, one (projection, 32-rank chunk) at a time while the stream runs. Parts of a unit from its kWH waves
// meet in LDS after the stream; split k and the epilogue are those of the decode kernel.
constexpr int kWWaves = 16;
constexpr int kWStream = 15;
constexpr int kWH = 3;                   // k-tiles per pass = stream waves per unit
constexpr int kWSlots = kWStream / kWH;  // units per workgroup (at most)
constexpr int kWPiece = kWave * 16;      // bytes of one load into LDS (16 per lane)
__host__ __device__ constexpr int wide_nbuf(int tmt) { return tmt <= 2 ? 4 : 2; }
__host__ __device__ constexpr int wide_frag_pieces(int tmt) { return kWH * tmt * 4; }
// a pass's buffer: its fragments [tt][j][s][lane], then one piece holding the tile scales [tt][j][16] (f32)
__host__ __device__ constexpr int wide_buf_bytes(int tmt) { return (wide_frag_pieces(tmt) + 1) * kWPiece; }
// loads into LDS per stream wave and pass (the spare ones go to a scratch piece, so every wave issues as many)
__host__ __device__ constexpr int wide_fills(int tmt) { return (wide_frag_pieces(tmt) + 1 + kWStream - 1) / kWStream; }

struct WideArgs {
  GemvArgs G;           // rows, chunks, part sums and counters as in the decode kernel (nu counts units)
  const u32x4* t_fin;   // LoRA-down t as bf16 hi/lo B-fragments, [p][tile][jc][hi, lo][lane] x 16 bytes
  int64_t t_fin_bytes;
};

template <int TMT, bool SILU, int LW>
__global__ void __launch_bounds__(kWWaves * kWave) k_wgemv(WideArgs wa) {
  constexpr int NR = SILU ? 2 : 1;
  constexpr int NB = wide_nbuf(TMT), LA = NB - 1;
  constexpr int UF = NB > LW + 1 ? NB : LW + 1;  // passes per loop step: buffers and weight slots stay constant indices
  static_assert(UF % NB == 0 && UF % (LW + 1) == 0 && LW >= LA, "pass pipeline");
  constexpr int kBuf = wide_buf_bytes(TMT), kFrag = wide_frag_pieces(TMT), kFills = wide_fills(TMT);
  constexpr int kTW = 2 * NR;  // weight loads per stream wave and pass
  constexpr int kOut = (kWSlots * TMT * 256 + kWWaves * kWave - 1) / (kWWaves * kWave);
  __shared__ __attribute__((aligned(16))) uint8_t s_b0[kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t s_b1[kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t s_b2[NB > 2 ? kBuf : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_b3[NB > 3 ? kBuf : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_spare[kWPiece];
  __shared__ __attribute__((aligned(16))) uint8_t s_lora[kWSlots * NR * TMT * kWPiece];  // LoRA-up [u][nr][tt][lane]
  __shared__ uint16_t s_res[kWSlots * TMT * 16 * 16];  // residual of each output (epilogue order)
  __shared__ ProjEpi s_pe[kMaxProj];
  __shared__ int s_last;
  auto buf = [&](int i) __attribute__((always_inline)) -> uint8_t* {  // (i is a constant wherever this is called)
    return i == 0 ? s_b0 : (i == 1 ? s_b1 : (i == 2 ? s_b2 : s_b3));
  };
  const GemvArgs& g = wa.G;
  const LinearArgs& a = g.L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const unsigned bid = blockIdx.x, nbr = (unsigned)g.nbr, nk = (unsigned)g.nk;
  const int b = (int)(bid % nbr), c = (int)(bid / nbr);
  const int KT = g.KT, ntiles = g.ntiles;
  const int u0 = (int)((unsigned)b * (unsigned)g.nu / nbr);
  const int U = (int)((unsigned)(b + 1) * (unsigned)g.nu / nbr) - u0;
  const int t0 = (int)((unsigned)c * (unsigned)KT / nk), T = (int)((unsigned)(c + 1) * (unsigned)KT / nk) - t0;
  const int ntl = ntiles < TMT ? ntiles : TMT;  // token tiles present (one launch covers every token)
  const int NP = (T + kWH - 1) / kWH;          // passes
  const bool stream_w = wave < kWStream;
  const int su = stream_w ? wave / kWH : 0, j = stream_w ? wave % kWH : 0;
  const bool live = stream_w && su < U;

  // epilogue parameters and the residual of this thread's outputs, requested before anything else (the stream waves'
  // wait counts below cover only the loads issued after them)
  if (threadIdx.x < kMaxProj) {
#pragma unroll
    for (int q = 0; q < kMaxProj; ++q)
      if (threadIdx.x == q && q < a.nproj) {
        const ProjArgs& P = a.p[q];
        s_pe[q] = ProjEpi{P.y, P.res, P.n, P.ldy, P.ld_res, gload(P.s_g), P.lambda, P.y_dtype, P.y_repeat,
                          P.head_dim, P.rg_begin, P.r};
      }
  }
  // (32-bit indices: rows and row strides are below 2^31; kept apart from the epilogue's 64-bit ones, which the
  // compiler would otherwise hold in registers across the stream)
  uint16_t res[kOut];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int e = threadIdx.x + i * kWWaves * kWave;
    const int u = (int)((unsigned)e / (TMT * 256)), tok = (e >> 4) & (TMT * 16 - 1), row = e & 15;
    const int gu = u0 + u;
    const uint16_t* rb = a.p[0].res;
    int rbeg = 0, nl = (int)a.p[0].n;
    uint32_t ld = (uint32_t)a.p[0].ld_res;
    if (!SILU) {
#pragma unroll
      for (int q = 1; q < kMaxProj; ++q)
        if (q < a.nproj && gu >= a.p[q].rg_begin) {
          rb = a.p[q].res;
          rbeg = a.p[q].rg_begin;
          nl = (int)a.p[q].n;
          ld = (uint32_t)a.p[q].ld_res;
        }
    }
    const int n = (gu - rbeg) * 16 + row;
    const bool ok = rb && u < U && tok < g.mt && n < nl;
    res[i] = gload(ok ? rb + ((size_t)((uint32_t)tok * ld) + (uint32_t)n) : reinterpret_cast<const uint16_t*>(a.xsc));
  }

  // weights of this wave's unit: k-tile t0 + q*kWH + j of pass q (past the chunk: out of range, reads 0)
  rsrc_t cd[NR], sd[NR];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    const int64_t gu = u0 + su;
    int p = nr;
    if (!SILU) {
      p = 0;
      for (int q = 1; q < a.nproj; ++q)
        if (gu >= a.p[q].rg_begin) p = q;
      p = __builtin_amdgcn_readfirstlane(p);
    }
    const ProjArgs& P = a.p[p];
    const int64_t rg = SILU ? gu : gu - P.rg_begin;
    const bool ok = live && rg * 16 < P.n;
    cd[nr] = make_rsrc(P.codes + rg * KT * kTileCodeBytes, ok ? KT * kTileCodeBytes : 0);
    sd[nr] = make_rsrc(P.scales + rg * KT * kTileScaleBytes, ok ? KT * kTileScaleBytes : 0);
  }
  const uint32_t c_off = lane * 16, s_off = ((lane % 16) * 2 + (lane / 16) / 2) * 4;
  auto wload = [&](GTile<NR>& t, int q) __attribute__((always_inline)) {
    const bool in = q * kWH + j < T;
    const int kt = t0 + q * kWH + j;
    const int kc = __builtin_amdgcn_readfirstlane(in ? kt * kTileCodeBytes : 0);
    const int ks = __builtin_amdgcn_readfirstlane(in ? kt * kTileScaleBytes : 0);
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      t.c[nr] = __builtin_amdgcn_raw_buffer_load_b128(cd[nr], in ? c_off : kOutOfRange, kc, kNonTemporal);
      t.sc[nr] = __builtin_amdgcn_raw_buffer_load_b32(sd[nr], in ? s_off : kOutOfRange, ks, kNonTemporal);
    }
  };
  // activations of pass q into LDS buffer dst: load slot i*kWStream + wave is fragment piece (tt, jj, s) =
  // (sl / (4*kWH), sl / 4 % kWH, sl % 4), then the scale piece, then spare loads (out of range, to the spare piece)
  const rsrc_t xsrc = make_rsrc(a.xs, (int64_t)ntl * KT * 4 * kWave * 16);
  const rsrc_t ssrc = make_rsrc(a.xsc, (int64_t)ntl * KT * 16 * 4);
  auto fill = [&](uint8_t* dst, int q) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kFills; ++i) {
      const int sl = i * kWStream + wave;
      if (sl < kFrag) {
        const int tt = sl / (4 * kWH), jj = (sl / 4) % kWH, s = sl % 4;
        const bool ok = q * kWH + jj < T && tt < ntl;
        const int so = __builtin_amdgcn_readfirstlane(ok ? ((tt * KT + t0 + q * kWH + jj) * 4 + s) * kWPiece : 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrc, (__attribute__((address_space(3))) void*)(dst + sl * kWPiece),
                                                 16, ok ? lane * 16 : kOutOfRange, so, 0, 0);
      } else if (sl == kFrag) {
        const int tt = lane / (4 * kWH), jj = (lane / 4) % kWH, qd = lane % 4;
        const bool ok = lane < TMT * kWH * 4 && q * kWH + jj < T && tt < ntl;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ssrc, (__attribute__((address_space(3))) void*)(dst + kFrag * kWPiece), 16,
            ok ? (uint32_t)(((tt * KT + t0 + q * kWH + jj) * 16 + qd * 4) * 4) : kOutOfRange, 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrc, (__attribute__((address_space(3))) void*)s_spare, 16,
                                                 kOutOfRange, 0, 0, 0);
      }
    }
  };

  f32x4 acc[NR][TMT];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr)
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) acc[nr][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // pass q from buffer B with weights t. A wave whose k-tile lies past the chunk has zero weights and reads the
  // pass's last k-tile in range (finite values), so it adds exactly zero.
  auto compute = [&](const uint8_t* B, const GTile<NR>& t, int q) __attribute__((always_inline)) {
    const int jl = T - q * kWH - 1;
    const int jj = j < jl ? j : jl;
    f32x4 part[NR][TMT];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt) part[nr][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 bf[TMT];
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt)
        bf[tt] = *reinterpret_cast<const u32x4*>(B + ((tt * kWH + jj) * 4 + s) * kWPiece + lane * 16);
#pragma unroll
      for (int nr = 0; nr < NR; ++nr) {
        const uint32_t scv = ((t.sc[nr] >> (8 * s)) & 0xFFu) * 0x00800080u;  // E4M3 byte << 7 = E4M3 * 2^-8 in f16
        const f16x2 sh = as_f16x2(scv);
        const uint32_t cw = t.c[nr][s];
        const f16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 0) * sh;
        const f16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 1) * sh;
        const f16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 2) * sh;
        const f16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 3) * sh;
        const f16x8 wv = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
#pragma unroll
        for (int tt = 0; tt < TMT; ++tt)
          part[nr][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, __builtin_bit_cast(f16x8, bf[tt]), part[nr][tt],
                                                                0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // one slice's fragments live at a time
    }
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) {
      const float u = *reinterpret_cast<const float*>(B + kFrag * kWPiece + ((tt * kWH + jj) * 16 + lane % 16) * 4);
#pragma unroll
      for (int nr = 0; nr < NR; ++nr)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[nr][tt][e] = __builtin_fmaf(part[nr][tt][e], u, acc[nr][tt][e]);
    }
  };

  // LoRA-up items of wave 15 (chunk 0 only): (projection p, rank chunk jc) over the block's units, in order. Item i:
  // the B rows of the units of projection p (16 rows x ranks jc*32 + 8 (lane/16) .. + 8) and t of every token tile.
  int pfirst = 0, nitems = 0;
  if (SILU) {
    nitems = a.nproj >= 2 ? (int)ceil_div(a.p[0].r, 32) + (int)ceil_div(a.p[1].r, 32) : 0;
  } else {
    int pl = 0;
    for (int q = 1; q < a.nproj; ++q) {
      if (u0 >= a.p[q].rg_begin) pfirst = q;
      if (u0 + U - 1 >= a.p[q].rg_begin) pl = q;
    }
    for (int q = pfirst; q <= pl; ++q) nitems += (int)ceil_div(a.p[q].r, 32);
  }
  const bool lora_w = wave == kWStream && c == 0;
  if (!lora_w) nitems = 0;
  nitems = __builtin_amdgcn_readfirstlane(nitems);
  auto item_of = [&](int it, int* p_out, int* jc_out) __attribute__((always_inline)) {
    int p = SILU ? 0 : pfirst, rem = it;
    for (int q = p; q < kMaxProj; ++q) {
      const int n = q < a.nproj ? (int)ceil_div(a.p[q].r, 32) : 0;
      if (rem < n) { p = q; break; }
      rem -= n;
    }
    *p_out = p;
    *jc_out = rem;
  };
  // (projection of unit gu from the kernel arguments: wave 15 works before any barrier has published s_pe)
  auto unit_proj_arg = [&](int gu) __attribute__((always_inline)) {
    int p = 0;
    for (int q = 1; q < a.nproj; ++q)
      if (gu >= a.p[q].rg_begin) p = q;
    return p;
  };
  struct LItem {
    u32x4 b[kWSlots], th[TMT], tl[TMT];
  };
  const rsrc_t tsrc = make_rsrc(wa.t_fin, wa.t_fin_bytes);
  auto item_issue = [&](LItem& L, int it) __attribute__((always_inline)) {
    int p, jc;
    item_of(it, &p, &jc);
    const ProjArgs* P = &a.p[0];
#pragma unroll
    for (int q = 1; q < kMaxProj; ++q)
      if (q == p) P = &a.p[q];
    const int r = P->r;
    const rsrc_t bsrc = make_rsrc(P->B, P->n * r * 2);
    const int nrows = (int)P->n;  // (n * r * 2 < 2^31: checked on the host)
#pragma unroll
    for (int u = 0; u < kWSlots; ++u) {
      const int gu = u0 + u;
      const bool mine = u < U && (SILU || unit_proj_arg(gu) == p);
      const int n = (SILU ? gu : gu - P->rg_begin) * 16 + lane % 16;
      const int j0 = jc * 32 + (lane / 16) * 8;
      if (r % 8 == 0) {
        L.b[u] = bload16(bsrc, (mine && n < nrows && j0 < r) ? (uint32_t)((n * r + j0) * 2) : kOutOfRange);
      } else {
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = (uint32_t)((n * r + j0 + 2 * e) * 2);
          const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
              bsrc, (mine && n < nrows && j0 + 2 * e < r) ? off : kOutOfRange, 0, 0);
          const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
              bsrc, (mine && n < nrows && j0 + 2 * e + 1 < r) ? off + 2 : kOutOfRange, 0, 0);
          w4[e] = lo | (hi << 16);
        }
        L.b[u] = u32x4{w4[0], w4[1], w4[2], w4[3]};
      }
    }
#pragma unroll
    for (int tt = 0; tt < TMT; ++tt) {
      const uint32_t off = (uint32_t)(((((int64_t)p * ntiles + tt) * kRankChunks + jc) * 2 * kWave + lane) * 16);
      L.th[tt] = bload16(tsrc, tt < ntl ? off : kOutOfRange);
      L.tl[tt] = bload16(tsrc, tt < ntl ? off + kWave * 16 : kOutOfRange);
    }
  };
  auto item_finish = [&](const LItem& L, int it) __attribute__((always_inline)) {
    int p, jc;
    item_of(it, &p, &jc);
    const int nr = SILU ? p : 0;
#pragma unroll
    for (int u = 0; u < kWSlots; ++u) {
      if (u >= U) break;
      if (!SILU && unit_proj_arg(u0 + u) != p) continue;
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt) {
        f32x4 la = {0.f, 0.f, 0.f, 0.f};
        la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, L.b[u]), __builtin_bit_cast(bf16x8, L.th[tt]),
                                                     la, 0, 0, 0);
        la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, L.b[u]), __builtin_bit_cast(bf16x8, L.tl[tt]),
                                                     la, 0, 0, 0);
        mfma_settle(la);
        f32x4* slot = reinterpret_cast<f32x4*>(s_lora + (((u * NR + nr) * TMT + tt) * kWave + lane) * 16);
        *slot = jc == 0 ? la : *slot + la;
      }
    }
  };

  // prologue: the first weight tiles and the first LA passes' activations, in the order of the pipeline: weights
  // W(0 .. LW-LA-1), then (fill(s), W(s + LW - LA)) for s < LA; each pass q then issues (fill(q + LA), W(q + LW)).
  // At the top of pass q the loads issued after fill(q) are W(q + LW - LA) and LA - 1 more (fill, W) pairs.
  GTile<NR> Wt[LW + 1];
  if (stream_w) {
#pragma unroll
    for (int s = 0; s < LW - LA; ++s) wload(Wt[s], s);
#pragma unroll
    for (int s = 0; s < LA; ++s) {
      fill(buf(s), s);
      wload(Wt[s + LW - LA], s + LW - LA);
    }
  }
#pragma unroll
  for (int i = 0; i < kOut; ++i) s_res[threadIdx.x + i * kWWaves * kWave] = res[i];
  constexpr int kWaitFill = vmcnt_imm(kTW + (LA - 1) * (kFills + kTW));

  // The stream waves and wave 15 run loops of their own with the same barriers (one per pass, UF passes per step),
  // so that the registers of the one are not held across the other's code.
  // (a plain barrier: a workgroup fence would also wait for the fills still in flight)
  if (stream_w) {
    for (int q0 = 0; q0 < NP; q0 += UF) {
#pragma unroll
      for (int i = 0; i < UF; ++i) {
        const int q = q0 + i;
        __builtin_amdgcn_s_waitcnt(kWaitFill);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        fill(buf((i + LA) % NB), q + LA);
        wload(Wt[(i + LW) % (LW + 1)], q + LW);
        __builtin_amdgcn_sched_barrier(0);
        if (live && q < NP) compute(buf(i % NB), Wt[i % (LW + 1)], q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // no load into LDS is in flight when the buffers are reused below
  } else {
    // wave 15: the first item before the first barrier (its memory round trip overlaps the stream waves' first
    // loads), then one per pass
    LItem L0;
    if (nitems > 0) item_issue(L0, 0);
    if (nitems > 0) item_finish(L0, 0);
    int it = 1;
    if (it < nitems) item_issue(L0, it);
    for (int q0 = 0; q0 < NP; q0 += UF) {
#pragma unroll
      for (int i = 0; i < UF; ++i) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (it < nitems) {
          item_finish(L0, it);
          if (++it < nitems) item_issue(L0, it);
        }
      }
    }
    for (; it < nitems; ++it) {  // items left when the passes are few
      item_finish(L0, it);
      if (it + 1 < nitems) item_issue(L0, it + 1);
    }
  }
  __syncthreads();

  // parts of phases 1 and 2 of each unit into buffers 0 and 1; phase 0 adds them (in phase order) and leaves the sum
  // in buffer 0
  auto part_slot = [&](uint8_t* B, int nr, int tt) __attribute__((always_inline)) {
    return reinterpret_cast<f32x4*>(B + ((((su * NR + nr) * TMT + tt) * kWave) + lane) * 16);
  };
  if (live && j > 0) {
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt) *part_slot(j == 1 ? s_b0 : s_b1, nr, tt) = acc[nr][tt];
  }
  __syncthreads();
  if (live && j == 0) {
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
      for (int tt = 0; tt < TMT; ++tt) {
        f32x4 v = acc[nr][tt] + *part_slot(s_b0, nr, tt);
        v += *part_slot(s_b1, nr, tt);
        *part_slot(s_b0, nr, tt) = v;
      }
  }
  __syncthreads();

  const bool has_lora = c == 0;  // LoRA terms were computed in chunk 0 (read only where the projection has an adapter)
  const int nout = U * TMT * 256;
  float vsum[kOut][NR], vlo[kOut][NR];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int e = threadIdx.x + i * kWWaves * kWave;
    const int u = (int)((unsigned)e / (TMT * 256)), tok = (e >> 4) & (TMT * 16 - 1), row = e & 15;
    const int tt = tok / 16, col = tok % 16;
    const int ln = (row / 4) * 16 + col, ii = row % 4;
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      float s = 0.f, lo = 0.f;
      if (e < nout) {
        s = reinterpret_cast<const float*>(s_b0 + ((((u * NR + nr) * TMT + tt) * kWave) + ln) * 16)[ii];
        if (has_lora && s_pe[SILU ? nr : unit_proj(s_pe, a.nproj, u0 + u)].r > 0)
          lo = reinterpret_cast<const float*>(s_lora + ((((u * NR + nr) * TMT + tt) * kWave) + ln) * 16)[ii];
      }
      vsum[i][nr] = s;
      vlo[i][nr] = lo;
    }
  }
  gemv_finish<TMT, SILU, kOut, kWWaves * kWave>(g, s_pe, s_res, &s_last, vsum, vlo, nout, b, c, u0);
}

// ------------------------------------------------------------------------------------------------------------------
// F: fused decode kernel for up to 16 tokens: the decode kernel above with the prologue folded in, one launch per
// call. Each workgroup builds the activation fragments of its own k-chunk in LDS from x, which it reads once into
// registers. With the norm (then the chunk is the whole row), the row statistics come from those registers in the
// standalone norm's summation order (running sums of the 256 stand-in threads kept in LDS, one round per 256 chunks of
// 8 channels), so h is bit for bit the norm's; the per-(token, k-tile) power-of-two exponents are the prologue's. When
// every token shares gamma + sigma * noise, the workgroup computes that scale once into LDS.
// The one step that needs all of a row's channels, the LoRA-down t = A h, is cut into items (projection, 32-rank
// chunk, k-chunk). Workgroup i computes item i from its LDS fragments (f16 * 2^-p gives back h exactly above 2^-32 of
// the tile's largest value) with 8 waves; its wave 15 adds their sums and stores the partial past the per-XCD caches,
// bit-inverted, so that a word of it reads zero until it is written: the partials are their own ready flags. Item i
// lives in workgroup i, workgroups are dispatched in index order and a producer waits for nothing before its item is
// out, so the waits below always end. The LoRA wave of a block's chunk-0 workgroup (a consumer) polls its projections'
// partials until every word is written (a wait bounded by a poll count: should it ever expire, the LoRA term becomes
// NaN, so the outputs show it, rather than the wave spinning on), adds them in k-chunk order and continues as in the
// decode kernel. The last consumer to finish its reads clears the partials and its counter, so they are zero between
// calls; they must be zero before the first.
constexpr int kFLoraWaves = 8;                                // waves computing a LoRA-down item
constexpr int kFRedBytes = kFLoraWaves * 2 * kWave * 16;      // their sums (top of LDS)
constexpr int kFMaxItems = kFusedItemsMax;
constexpr int kFItemTiles = 4;                                // k-tiles per LoRA-down item without a split k
constexpr uint32_t kFSpin = 1u << 24;                         // polls before a wait gives up (about a second)
__host__ __device__ constexpr int fused_lds_top(int nr) {     // LDS bytes above the fragments and tile scales
  return gemv_lred_bytes(nr, 1) > kFRedBytes ? gemv_lred_bytes(nr, 1) : kFRedBytes;
}

struct FusedArgs {
  GemvArgs G;
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* gamma;
  const float* noise;
  int64_t noise_ld;
  float sigma, eps;
  QnDraw draw;
  int32_t g_shared;         // with the norm: every token has the same gamma + sigma * noise
  int32_t ctl_k;            // k-tiles per LoRA-down item when nk == 1 (0 with a split k: an item is a whole chunk)
  int32_t nkc;              // LoRA-down k-chunks per (projection, rank chunk)
  int32_t nitems;           // items, in (projection, rank chunk, k-chunk) order; item i = workgroup i
  int32_t pair0[kMaxProj];  // first (projection, rank chunk) pair of each projection
  float* t_part;            // [item][lane][8] f32 partials, in the LoRA-up B-fragment lane order
  uint32_t* ctl;            // consumers past their reads (one word)
};

// x * rstd * g rounded to bf16, g = gamma + sigma * noise already formed (the same operations as aqn_value).
__device__ __forceinline__ uint32_t aqn_scaled(float x, float rstd, float g) {
  return f32_to_bf16(__fmul_rn(__fmul_rn(x, rstd), g));
}

// GSH (with the norm): every token has the same gamma + sigma * noise (FusedArgs::g_shared).
template <bool SILU, bool AQN, bool VEC, bool GSH>
__global__ void __launch_bounds__(kGWaves * kWave) k_fgemv(FusedArgs f) {
  constexpr int NR = SILU ? 2 : 1, D = 3;
  constexpr int kOut = (kGMaxUnits * 16 * 16 + kGWaves * kWave - 1) / (kGWaves * kWave);
  constexpr int kAPre = 2;  // A fragments per item wave requested up front (an item of 4 k-tiles needs 2)
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kGLds];
  __shared__ uint16_t s_res[kGMaxUnits * 16 * 16];
  __shared__ ProjEpi s_pe[kMaxProj];
  __shared__ float s_rstd[16];
  __shared__ int s_last;
  const GemvArgs& g = f.G;
  const LinearArgs& a = g.L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const unsigned bid = blockIdx.x, nbr = (unsigned)g.nbr, nk = (unsigned)g.nk;
  const int b = (int)(bid / nk), c = (int)(bid % nk);  // chunks of a block adjacent: item i <-> workgroup i
  const int KT = g.KT, mt = g.mt, k = (int)a.k;
  const int u0 = (int)((unsigned)b * (unsigned)g.nu / nbr);
  const int U = (int)((unsigned)(b + 1) * (unsigned)g.nu / nbr) - u0;
  const int t0 = (int)((unsigned)c * (unsigned)KT / nk), T = (int)((unsigned)(c + 1) * (unsigned)KT / nk) - t0;
  uint8_t* const lred = s_lds + kGLds - gemv_lred_bytes(NR, 1);
  const int fr_bytes = T * 4 * kWave * 16;
  const int kc0 = t0 * kKTile;   // first channel of the chunk
  constexpr bool gsh = AQN && GSH;

  // stream waves: unit su, k-part sj of the chunk (as in the decode kernel; here h = 15 / U is computed, not looked
  // up: a table in memory is a load, and its wait would come after every load issued before it)
  const int h = U > 0 ? kGStream / U : 1;
  const bool streams = wave < U * h;
  const int su = streams ? (int)((unsigned)wave / (unsigned)h) : 0, sj = streams ? wave - su * h : 0;
  const int ta = __builtin_amdgcn_readfirstlane(t0 + (int)((unsigned)(sj * T) / (unsigned)h));
  const int tb = __builtin_amdgcn_readfirstlane(streams ? t0 + (int)((unsigned)((sj + 1) * T) / (unsigned)h) : ta);
  rsrc_t cd[NR], sd[NR];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) {
    const int64_t gu = u0 + su;
    int p = nr;
    if (!SILU) {
      p = 0;
      for (int q = 1; q < a.nproj; ++q)
        if (gu >= a.p[q].rg_begin) p = q;
      p = __builtin_amdgcn_readfirstlane(p);
    }
    const ProjArgs& P = a.p[p];
    const int64_t rg = SILU ? gu : gu - P.rg_begin;
    const bool live = streams && rg * 16 < P.n;
    cd[nr] = make_rsrc(P.codes + rg * KT * kTileCodeBytes, live ? KT * kTileCodeBytes : 0);
    sd[nr] = make_rsrc(P.scales + rg * KT * kTileScaleBytes, live ? KT * kTileScaleBytes : 0);
  }
  const uint32_t c_off = lane * 16, s_off = ((lane % 16) * 2 + (lane / 16) / 2) * 4;
  auto load = [&](GTile<NR>& tl, int kt) {
    const bool in = kt < tb;
    const int kc = __builtin_amdgcn_readfirstlane(in ? kt * kTileCodeBytes : 0);
    const int ks = __builtin_amdgcn_readfirstlane(in ? kt * kTileScaleBytes : 0);
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      tl.c[nr] = __builtin_amdgcn_raw_buffer_load_b128(cd[nr], in ? c_off : kOutOfRange, kc, kNonTemporal);
      tl.sc[nr] = __builtin_amdgcn_raw_buffer_load_b32(sd[nr], in ? s_off : kOutOfRange, ks, kNonTemporal);
    }
  };
  // tensor scales of the projections (threads 0..nproj-1), to LDS below
  float sg_mine = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxProj; ++q)
    if (threadIdx.x == q && q < a.nproj) sg_mine = gload(a.p[q].s_g);
  // ---- requests, in the order they are needed: the shared norm scale's inputs, x, residuals, the LoRA-down item's
  //      A fragments, the first weight tiles (the waits for earlier ones then leave the later ones in flight)
  const rsrc_t gsrc = make_rsrc(f.gamma, AQN ? (int64_t)k * 2 : 0);
  const rsrc_t zsrc = make_rsrc(f.noise, (AQN && f.noise) ? ((int64_t)(mt - 1) * f.noise_ld + k) * 4 : 0);
  uint32_t gw[4] = {0u, 0u, 0u, 0u};
  float gz[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (gsh) {  // channels kc0 + 8 tid .. + 8 (one group per thread: a chunk has at most 31 * 16 groups)
    const int kk = kc0 + (int)threadIdx.x * 8;
    const bool ok = (int)threadIdx.x < T * 16 && kk < k;
    bload_bf16x8<VEC>(gsrc, ok ? (uint32_t)kk * 2 : kOutOfRange, gw);
    if (!f.draw.on) bload_f32x8<VEC>(zsrc, ok ? (uint32_t)kk * 4 : kOutOfRange, gz);
  }
  // unit (token t, local k-tile lt, channel quarter jq) of pass ps: t = lane % 16, jq = lane / 16, lt = wave + 16 ps; it
  // holds channels 32 jq .. 32 jq + 31 of the k-tile, four groups of 8. A wave covers one k-tile of all 16 tokens, so a
  // (token, k-tile) spans four lanes 16 apart, and its fragment stores go to 16 distinct LDS bank groups per 16 lanes.
  const int ut = lane % 16, uq = lane / 16;
  const rsrc_t xsrc = make_rsrc(f.x, ((int64_t)(mt - 1) * f.ldx + k) * 2);
  uint32_t hx[2][4][4];
#pragma unroll
  for (int ps = 0; ps < 2; ++ps)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lt = wave + 16 * ps, kk = kc0 + lt * kKTile + uq * 32 + i * 8;
      const bool ok = ut < mt && lt < T && kk < k;
      bload_bf16x8<VEC>(xsrc, ok ? (uint32_t)(((int64_t)ut * f.ldx + kk) * 2) : kOutOfRange, hx[ps][i]);
    }
  // residual of this thread's outputs (output e = (unit, token, row) = ((u * 16 + tok) * 16 + row)); outputs without
  // one read a valid stand-in address (x)
  uint16_t res[kOut];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int e = threadIdx.x + i * kGWaves * kWave;
    const int u = e >> 8, tok = (e >> 4) & 15, row = e & 15;
    const int64_t gu = u0 + u;
    const uint16_t* rb = a.p[0].res;
    int64_t rbeg = 0, nl = a.p[0].n, ld = a.p[0].ld_res;
    if (!SILU) {
#pragma unroll
      for (int q = 1; q < kMaxProj; ++q)
        if (q < a.nproj && gu >= a.p[q].rg_begin) {
          rb = a.p[q].res;
          rbeg = a.p[q].rg_begin;
          nl = a.p[q].n;
          ld = a.p[q].ld_res;
        }
    }
    const int64_t n = (gu - rbeg) * 16 + row;
    const bool ok = rb && u < U && tok < mt && n < nl;
    res[i] = gload(ok ? rb + tok * ld + n : f.x);
  }
  // this workgroup's LoRA-down item, if it has one: (projection ip, rank chunk ijc), local k-tiles [lt0, lt0 + ltn)
  const bool producer = (int)bid < f.nitems;
  int ip = 0, ijc = 0, lt0 = 0, ltn = 0;
  if (producer) {
    const int pair = (int)bid / f.nkc, kc = (int)bid % f.nkc;
#pragma unroll
    for (int q = 1; q < kMaxProj; ++q)
      if (q < a.nproj && pair >= f.pair0[q]) ip = q;
    ijc = pair - f.pair0[ip];
    lt0 = f.ctl_k > 0 ? kc * f.ctl_k : 0;
    ltn = f.ctl_k > 0 ? (T - lt0 < f.ctl_k ? T - lt0 : f.ctl_k) : T;
  }
  const uint16_t* Ap = nullptr;
  int ir = 0;
#pragma unroll
  for (int q = 0; q < kMaxProj; ++q)
    if (q == ip) {
      Ap = a.p[q].A;
      ir = a.p[q].r;
    }
  const rsrc_t asrc = make_rsrc(Ap, producer ? (int64_t)ir * k * 2 : 0);
  // A fragment of (slice sl, half gh) for waves 0..7: ranks jc*32 + 16 gh + lane%16, k of the slice + 8 (lane/16)
  auto a_off = [&](int sl, int gh) -> uint32_t {
    const int j = ijc * 32 + gh * 16 + lane % 16;
    const int kk = (t0 + lt0 + sl / 4) * kKTile + (sl % 4) * 32 + (lane / 16) * 8;
    const bool ok = producer && wave < kFLoraWaves && sl < ltn * 4 && j < ir && kk < k;
    return ok ? (uint32_t)(((int64_t)j * k + kk) * 2) : kOutOfRange;
  };
  u32x4 apre[kAPre][2];
#pragma unroll
  for (int i = 0; i < kAPre; ++i)
#pragma unroll
    for (int gh = 0; gh < 2; ++gh) apre[i][gh] = bload16(asrc, a_off(wave + i * kFLoraWaves, gh));
  // the first D - 1 weight tiles of the stream waves
  GTile<NR> Bt[D];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < D - 1; ++j) {
    load(Bt[j], ta + j);
    __builtin_amdgcn_sched_barrier(0);  // issue order of the first tiles: the loop's wait counts rely on it
  }

  if (threadIdx.x < kMaxProj) {
#pragma unroll
    for (int q = 0; q < kMaxProj; ++q)
      if (threadIdx.x == q && q < a.nproj) {
        const ProjArgs& P = a.p[q];
        s_pe[q] = ProjEpi{P.y, P.res, P.n, P.ldy, P.ld_res, sg_mine, P.lambda, P.y_dtype, P.y_repeat, P.head_dim,
                          P.rg_begin, P.r};
      }
  }
  // the shared norm scale g = gamma + sigma * noise of the chunk's channels, f32, at the top of LDS (below it the
  // fragments; the LoRA-down sums and LoRA slots reuse it later)
  float* const s_g = reinterpret_cast<float*>(s_lds + kGLds - T * kKTile * 4);
  if (gsh && (int)threadIdx.x < T * 16) {
    if (f.draw.on) aqn_noise8(f.draw, draw_index(f.draw, 0), (uint64_t)(kc0 / 8 + threadIdx.x), gz);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s_g[threadIdx.x * 8 + 2 * e] = __fadd_rn(lo_bf16(gw[e]), __fmul_rn(f.sigma, gz[2 * e]));
      s_g[threadIdx.x * 8 + 2 * e + 1] = __fadd_rn(hi_bf16(gw[e]), __fmul_rn(f.sigma, gz[2 * e + 1]));
    }
  }

  // 1. with the norm (the chunk is the whole row): per token, the standalone norm's sum of squares. Stand-in thread s
  //    (of 256) adds the chunks c = s, s + 256, ... of 8 channels in order, elements in order; its running sum sits in
  //    LDS slot [s][token] between rounds: round 0 is pass 0 (chunks 0..255), round 1 pass 1 (the rest; a row has at
  //    most 31 * 16 chunks). Then wave t adds token t's 256 stand-ins as four wave sums taken in order.
  if (AQN) {
    float* const s_ss = reinterpret_cast<float*>(s_lds);  // [256][16] (in the fragment area, written later)
    for (int i = threadIdx.x; i < 256 * 16; i += kGWaves * kWave)
      if (i / 16 >= T * 16) s_ss[i] = 0.0f;  // stand-ins without a chunk
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int lt = wave + 16 * ps;
      if (ps == 1 && T <= 16) break;
      if (lt < T) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sl = (lt % 16) * 16 + uq * 4 + i;  // stand-in of chunk lt * 16 + uq * 4 + i
          float s = ps == 0 ? 0.0f : s_ss[sl * 16 + ut];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = lo_bf16(hx[ps][i][e]), x1 = hi_bf16(hx[ps][i][e]);
            s = __fadd_rn(s, __fmul_rn(x0, x0));
            s = __fadd_rn(s, __fmul_rn(x1, x1));
          }
          s_ss[sl * 16 + ut] = s;
        }
      }
      __syncthreads();
    }
    if (wave < mt) {
      float tot = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) tot = __fadd_rn(tot, wave_sum(s_ss[(v * kWave + lane) * 16 + wave]));
      if (lane == 0) s_rstd[wave] = rms_rstd(tot, k, f.eps);
    }
    __syncthreads();
  }

  // 2. h of every unit (from the registers), the (token, k-tile) exponent (amax over the unit's 32 values and the
  //    three other lanes of the token) and the fragments: [lt][s][lane] 16 bytes, then [lt][16] f32 tile scales 2^-p
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    const int lt = wave + 16 * ps;
    if (lt >= T) break;  // (uniform)
    uint32_t hv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[i][e] = hx[ps][i][e];
    if (AQN && ut < mt) {
      const float rstd = s_rstd[ut];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = lt * 16 + uq * 4 + i, kk = kc0 + ch * 8;
        if (kk >= k) continue;
        float gv[8];
        if (gsh) {
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(s_g + ch * 8);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(s_g + ch * 8 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gv[e] = g0[e];
            gv[4 + e] = g1[e];
          }
        } else {  // a scale of its own per token: gamma and this token's noise (read or drawn), one group at a time
          uint32_t gb[4];
          float z[8];
          __builtin_amdgcn_sched_barrier(0);
          bload_bf16x8<VEC>(gsrc, (uint32_t)kk * 2, gb);
          if (f.draw.on) aqn_noise8(f.draw, draw_index(f.draw, ut), (uint64_t)(kk / 8), z);
          else bload_f32x8<VEC>(zsrc, (uint32_t)((ut * f.noise_ld + kk) * 4), z);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gv[2 * e] = __fadd_rn(lo_bf16(gb[e]), __fmul_rn(f.sigma, z[2 * e]));
            gv[2 * e + 1] = __fadd_rn(hi_bf16(gb[e]), __fmul_rn(f.sigma, z[2 * e + 1]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hv[i][e] = aqn_scaled(lo_bf16(hv[i][e]), rstd, gv[2 * e]) |
                     (aqn_scaled(hi_bf16(hv[i][e]), rstd, gv[2 * e + 1]) << 16);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(hv[i][e])), fabsf(hi_bf16(hv[i][e]))));
    amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
    const int pw = act_exponent(amax);
    const float up = __uint_as_float((uint32_t)(pw + 127) << 23);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f16x2 v;
        v[0] = (_Float16)__fmul_rn(lo_bf16(hv[i][e]), up);
        v[1] = (_Float16)__fmul_rn(hi_bf16(hv[i][e]), up);
        packed[e] = __builtin_bit_cast(uint32_t, v);
      }
      // group jj = 4 uq + i: slice s = uq, lane group i
      *reinterpret_cast<u32x4*>(s_lds + ((lt * 4 + uq) * kWave + i * 16 + ut) * 16) =
          u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
    if (uq == 0)
      *reinterpret_cast<float*>(s_lds + fr_bytes + (lt * 16 + ut) * 4) = __uint_as_float((uint32_t)(127 - pw) << 23);
  }
#pragma unroll
  for (int i = 0; i < kOut; ++i) s_res[threadIdx.x + i * kGWaves * kWave] = res[i];
  __syncthreads();

  // 3. the LoRA-down item: waves 0..7 over its 32-wide k-slices (B-fragment = h back from the f16 fragment, token
  //    lane%16), two bf16 MFMAs per slice, into LDS; wave 15 adds the eight waves' sums in wave order, stores the
  //    partial past the caches in the LoRA-up's lane order
  if (producer) {
    f32x4* s_red = reinterpret_cast<f32x4*>(s_lds + kGLds - kFRedBytes);
    if (wave < kFLoraWaves) {
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      for (int i0 = 0; i0 * kFLoraWaves < ltn * 4; i0 += kAPre) {
        u32x4 af[kAPre][2];
        if (i0 == 0) {
#pragma unroll
          for (int i = 0; i < kAPre; ++i) af[i][0] = apre[i][0], af[i][1] = apre[i][1];
        } else {
#pragma unroll
          for (int i = 0; i < kAPre; ++i)
#pragma unroll
            for (int gh = 0; gh < 2; ++gh) af[i][gh] = bload16(asrc, a_off(wave + (i0 + i) * kFLoraWaves, gh));
        }
#pragma unroll
        for (int i = 0; i < kAPre; ++i) {
          const int sl = wave + (i0 + i) * kFLoraWaves;
          if (sl >= ltn * 4) break;
          const int lt = lt0 + sl / 4, s = sl % 4;
          const u32x4 fr = *reinterpret_cast<const u32x4*>(s_lds + ((lt * 4 + s) * kWave + lane) * 16);
          const float dn = *reinterpret_cast<const float*>(s_lds + fr_bytes + (lt * 16 + lane % 16) * 4);
          uint32_t hb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f16x2 v = as_f16x2(fr[e]);
            hb[e] = (uint32_t)f32_to_bf16(__fmul_rn((float)v[0], dn)) |
                    ((uint32_t)f32_to_bf16(__fmul_rn((float)v[1], dn)) << 16);
          }
          const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{hb[0], hb[1], hb[2], hb[3]});
#pragma unroll
          for (int gh = 0; gh < 2; ++gh)
            acc[gh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i][gh]), bv, acc[gh], 0,
                                                              0, 0);
        }
      }
      mfma_settle(acc[0]);  // (the loop's exit separates the MFMAs from these stores)
      mfma_settle(acc[1]);
      s_red[(wave * 2 + 0) * kWave + lane] = acc[0];
      s_red[(wave * 2 + 1) * kWave + lane] = acc[1];
    }
    __syncthreads();
    if (wave == kGWaves - 1) {
      // lane L = (jl / 8) * 16 + token holds ranks jl = 8 (L / 16) .. + 7 of the chunk; rank jl's sum sits in D lane
      // ((jl % 16) / 4) * 16 + token, element jl % 4, of half jl / 16
      const int tok = lane % 16;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jl = (lane / 16) * 8 + e, gh = jl / 16, jr = jl % 16;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kFLoraWaves; ++w) sum += s_red[(w * 2 + gh) * kWave + (jr / 4) * 16 + tok][jr % 4];
        v[e] = sum;
      }
      // stored bit-inverted: a word reads 0 until written (an all-ones f32, a NaN no arithmetic produces, is the
      // only value that would store as 0)
      const rsrc_t tsrc = make_rsrc(f.t_part, (int64_t)f.nitems * kWave * 32);
      const uint32_t off = (uint32_t)(((int64_t)bid * kWave + lane) * 32);
      u32x4 w0, w1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = ~__float_as_uint(v[e]);
        w1[e] = ~__float_as_uint(v[4 + e]);
      }
      __builtin_amdgcn_raw_buffer_store_b128(w0, tsrc, off, 0, kCoherent);
      __builtin_amdgcn_raw_buffer_store_b128(w1, tsrc, off + 16, 0, kCoherent);
    }
  }

  // 4. the weight stream (as in the decode kernel)
  f32x4 acc[NR];
#pragma unroll
  for (int nr = 0; nr < NR; ++nr) acc[nr] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const GTile<NR>& tl, int kt) {
    const int lt = (kt < tb ? kt : tb - 1) - t0;
    f32x4 part[NR];
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) part[nr] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 bf = *reinterpret_cast<const u32x4*>(s_lds + ((lt * 4 + s) * kWave + lane) * 16);
#pragma unroll
      for (int nr = 0; nr < NR; ++nr) {
        const uint32_t scv = ((tl.sc[nr] >> (8 * s)) & 0xFFu) * 0x00800080u;  // E4M3 byte << 7 = E4M3 * 2^-8 in f16
        const f16x2 sh = __builtin_bit_cast(f16x2, scv);
        const uint32_t cw = tl.c[nr][s];
        const f16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 0) * sh;
        const f16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 1) * sh;
        const f16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 2) * sh;
        const f16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 3) * sh;
        const f16x8 wv = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
        part[nr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, __builtin_bit_cast(f16x8, bf), part[nr], 0, 0, 0);
      }
    }
    const float u = *reinterpret_cast<const float*>(s_lds + fr_bytes + (lt * 16 + lane % 16) * 4);
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[nr][e] = __builtin_fmaf(part[nr][e], u, acc[nr][e]);
  };
  if (streams) {
    for (int kt = ta; kt < tb; kt += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        load(Bt[(j + D - 1) % D], kt + j + D - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(Bt[j], kt + j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // 5. LoRA-up of the block's rows (chunk-0 workgroup, wave 15): per projection and rank chunk, the partials of its
  //    k-chunk items (polled until written) added in k-chunk order, split into bf16 hi and lo, two MFMAs per unit.
  //    Past its reads the wave counts itself; the last consumer clears the partials and the count for the next call.
  if (wave == kGWaves - 1 && c == 0) {
    const rsrc_t tsrc = make_rsrc(f.t_part, (int64_t)f.nitems * kWave * 32);
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      int pfirst = SILU ? nr : unit_proj(s_pe, a.nproj, u0), plast = SILU ? nr : unit_proj(s_pe, a.nproj, u0 + U - 1);
      pfirst = __builtin_amdgcn_readfirstlane(pfirst);
      plast = __builtin_amdgcn_readfirstlane(plast);
      for (int p = pfirst; p <= plast; ++p) {
        const ProjEpi& E = s_pe[p];
        const uint16_t* Bm = nullptr;
        int pr0 = 0;
#pragma unroll
        for (int q = 0; q < kMaxProj; ++q)
          if (q == p) {
            Bm = a.p[q].B;
            pr0 = f.pair0[q];
          }
        const int r = E.r;
        for (int jc = 0; jc * 32 < r; ++jc) {
          const rsrc_t bsrc = make_rsrc(Bm, E.n * r * 2);
          u32x4 bfr[kGMaxUnits];
#pragma unroll
          for (int u = 0; u < kGMaxUnits; ++u) {
            const bool mine = u < U && (SILU || unit_proj(s_pe, a.nproj, u0 + u) == p);
            const int64_t n = (SILU ? u0 + u : u0 + u - E.rg_begin) * 16 + lane % 16;
            const int j0 = jc * 32 + (lane / 16) * 8;
            if (r % 8 == 0) {
              bfr[u] = bload16(bsrc, (mine && n < E.n && j0 < r) ? (uint32_t)((n * r + j0) * 2) : kOutOfRange);
            } else {
              uint32_t w[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int64_t off = (n * r + j0 + 2 * e) * 2;
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                    bsrc, (mine && n < E.n && j0 + 2 * e < r) ? (uint32_t)off : kOutOfRange, 0, 0);
                const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                    bsrc, (mine && n < E.n && j0 + 2 * e + 1 < r) ? (uint32_t)(off + 2) : kOutOfRange, 0, 0);
                w[e] = lo | (hi << 16);
              }
              bfr[u] = u32x4{w[0], w[1], w[2], w[3]};
            }
          }
          // the partials of (p, jc)'s k-chunk items i0 .. i0 + nkc - 1, four per batch of loads, polled until every word
          // is written (non-zero) and added in item order; a batch that never completes within the poll limit gives NaN
          const int i0 = (pr0 + jc) * f.nkc;
          constexpr int kTB = 4;
          bool ready = true;
          f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
          for (int kc0 = 0; kc0 < f.nkc; kc0 += kTB) {
            u32x4 q[kTB][2];
            bool got = false;
            for (uint32_t spins = 0; spins < kFSpin && !got; ++spins) {
              if (spins > 0) __builtin_amdgcn_s_sleep(2);
              bool all = true;
#pragma unroll
              for (int v = 0; v < kTB; ++v) {
                const bool in = kc0 + v < f.nkc;
                const uint32_t off = (uint32_t)(((int64_t)(i0 + kc0 + v) * kWave + lane) * 32);
                q[v][0] = __builtin_amdgcn_raw_buffer_load_b128(tsrc, in ? off : kOutOfRange, 0, kCoherent);
                q[v][1] = __builtin_amdgcn_raw_buffer_load_b128(tsrc, in ? off + 16 : kOutOfRange, 0, kCoherent);
              }
#pragma unroll
              for (int v = 0; v < kTB; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  all = all && (kc0 + v >= f.nkc || (q[v][0][e] != 0u && q[v][1][e] != 0u));
              got = __all(all) != 0;
            }
            ready = ready && got;
#pragma unroll
            for (int v = 0; v < kTB; ++v) {
              if (kc0 + v >= f.nkc) break;
              f32x4 a, b;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                a[e] = __uint_as_float(~q[v][0][e]);
                b[e] = __uint_as_float(~q[v][1][e]);
              }
              s0 += a;
              s1 += b;
            }
          }
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float t = ready ? (e < 4 ? s0[e] : s1[e - 4]) : __uint_as_float(0x7fc00000u);
            const uint32_t th = f32_to_bf16(t);
            const uint32_t tl = f32_to_bf16(t - bf16_to_f32((uint16_t)th));  // t - th is exact in f32
            if (e % 2 == 0) {
              hi[e / 2] = th;
              lo[e / 2] = tl;
            } else {
              hi[e / 2] |= th << 16;
              lo[e / 2] |= tl << 16;
            }
          }
          const u32x4 thi = u32x4{hi[0], hi[1], hi[2], hi[3]}, tlo = u32x4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
          for (int u = 0; u < kGMaxUnits; ++u) {
            if (u >= U) break;
            if (!SILU && unit_proj(s_pe, a.nproj, u0 + u) != p) continue;
            f32x4 la = {0.f, 0.f, 0.f, 0.f};
            la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr[u]),
                                                         __builtin_bit_cast(bf16x8, thi), la, 0, 0, 0);
            la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr[u]),
                                                         __builtin_bit_cast(bf16x8, tlo), la, 0, 0, 0);
            mfma_settle(la);  // (the store below sits behind a branch on one of its paths)
            f32x4* slot = reinterpret_cast<f32x4*>(lred + ((u * NR + nr) * kWave + lane) * 16);
            *slot = jc == 0 ? la : *slot + la;
          }
        }
      }
    }
    // every read of this consumer is done: count it; the last one clears the partials and the count
    uint32_t done = 0;
    if (lane == 0) done = __hip_atomic_fetch_add(f.ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    done = __shfl(done, 0, kWave);
    if (done == nbr - 1) {
      for (int i = 0; i < f.nitems * 2; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, tsrc, (uint32_t)((i * kWave + lane) * 16), 0,
                                               kCoherent);
      if (lane == 0) __hip_atomic_store(f.ctl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();  // every wave is done with the activations in LDS

  // 6. part sums of the stream waves into LDS (over the activation area), then the per-output sums
  if (streams) {
#pragma unroll
    for (int nr = 0; nr < NR; ++nr)
      *reinterpret_cast<f32x4*>(s_lds + (((su * h + sj) * NR + nr) * kWave + lane) * 16) = acc[nr];
  }
  __syncthreads();
  const bool has_lora = c == 0;
  const int nout = U * 256;
  float vsum[kOut][NR], vlo[kOut][NR];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int e = threadIdx.x + i * kGWaves * kWave;
    const int u = e >> 8, tok = (e >> 4) & 15, row = e & 15;
    const int ln = (row / 4) * 16 + tok, ii = row % 4;
#pragma unroll
    for (int nr = 0; nr < NR; ++nr) {
      float s = 0.f, lo = 0.f;
      if (e < nout) {
        for (int j = 0; j < h; ++j)
          s += reinterpret_cast<const float*>(s_lds + (((u * h + j) * NR + nr) * kWave + ln) * 16)[ii];
        if (has_lora && s_pe[SILU ? nr : unit_proj(s_pe, a.nproj, u0 + u)].r > 0)
          lo = reinterpret_cast<const float*>(lred + ((u * NR + nr) * kWave + ln) * 16)[ii];
      }
      vsum[i][nr] = s;
      vlo[i][nr] = lo;
    }
  }
  // 7. split k: as in the decode kernel
  bool epilogue = true;
  if (g.nk > 1) {
    const int64_t PB = gemv_block_floats(NR, 1);
    float* pb = g.pbuf + (int64_t)b * (g.nk + 1) * PB;
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int e = threadIdx.x + i * kGWaves * kWave;
      if (e >= nout) break;
#pragma unroll
      for (int nr = 0; nr < NR; ++nr) {
        __hip_atomic_store(pb + (int64_t)c * PB + (int64_t)e * NR + nr, vsum[i][nr], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (c == 0)
          __hip_atomic_store(pb + (int64_t)g.nk * PB + (int64_t)e * NR + nr, vlo[i][nr], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(g.cnt + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (uint32_t)(g.nk - 1);
    __syncthreads();
    epilogue = s_last != 0;
    if (epilogue) {
      constexpr int kRedBatch = 8;
#pragma unroll
      for (int i = 0; i < kOut; ++i)
#pragma unroll
        for (int nr = 0; nr < NR; ++nr) vsum[i][nr] = 0.f;
      for (int c0 = 0; c0 < g.nk; c0 += kRedBatch) {
        float q[kOut][NR][kRedBatch];
#pragma unroll
        for (int i = 0; i < kOut; ++i) {
          const int e = threadIdx.x + i * kGWaves * kWave;
#pragma unroll
          for (int nr = 0; nr < NR; ++nr)
#pragma unroll
            for (int v = 0; v < kRedBatch; ++v)
              q[i][nr][v] = (e < nout && c0 + v < g.nk)
                                ? __hip_atomic_load(pb + (int64_t)(c0 + v) * PB + (int64_t)e * NR + nr,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : 0.f;
          if (c0 == 0) {
#pragma unroll
            for (int nr = 0; nr < NR; ++nr)
              vlo[i][nr] = e < nout ? __hip_atomic_load(pb + (int64_t)g.nk * PB + (int64_t)e * NR + nr,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                    : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < kOut; ++i)
#pragma unroll
          for (int nr = 0; nr < NR; ++nr)
#pragma unroll
            for (int v = 0; v < kRedBatch; ++v) {
              if (c0 + v >= g.nk) break;
              vsum[i][nr] = (c0 + v == 0) ? q[i][nr][v] : vsum[i][nr] + q[i][nr][v];
            }
      }
      if (threadIdx.x == 0) __hip_atomic_store(g.cnt + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // 8. epilogue: y = s_g * sum + lambda * lora (SILU: SiLU(gate) * up), + residual, broadcast, rounding
  if (epilogue) {
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int e = threadIdx.x + i * kGWaves * kWave;
      if (e >= nout) break;
      const int u = e >> 8, tok = (e >> 4) & 15, row = e & 15;
      if (tok >= mt) continue;
      const int64_t gu = u0 + u;
      const int p0 = SILU ? 0 : unit_proj(s_pe, a.nproj, gu);
      const ProjEpi& E = s_pe[p0];
      const int64_t n = (SILU ? gu : gu - E.rg_begin) * 16 + row;
      if (n >= E.n) continue;
      float val[NR];
#pragma unroll
      for (int nr = 0; nr < NR; ++nr) {
        const ProjEpi& F = s_pe[SILU ? nr : p0];
        val[nr] = F.sg * vsum[i][nr] + F.lambda * vlo[i][nr];
      }
      float out = val[0];
      if (SILU) out = val[0] / (1.0f + __expf(-val[0])) * val[NR - 1];
      if (E.res) out += bf16_to_f32(s_res[e]);
      store_output(E.y, E.y_dtype, (int64_t)tok * E.ldy, n, E.y_repeat, E.head_dim, out);
    }
  }
}

// Row blocks x k-chunks of the decode kernel: about one workgroup per CU, at most kGMaxUnits units per block, the
// chunk's activations within LDS; among those, the cut with the least estimated time (largest share streamed at
// ~25 GB/s per CU, the activation copy at ~80 GB/s, ~1.5 us more for a split k).
struct GemvCut {
  int nbr, nk;
};
// k-tiles of activations a workgroup of the decode kernel can hold in LDS
inline int64_t gemv_act_cap(int tmt, int nr) { return (kGLds - gemv_lred_bytes(nr, tmt)) / ((int64_t)tmt * kGTileAct); }

// nk_only > 0: only that many k-chunks (a cut asked for by the caller's options). act_cap: k-tiles of activations a
// workgroup holds (at most).
inline GemvCut gemv_cut(int64_t nu, int64_t KT, int tmt, int nr, int nk_only, int64_t act_cap) {
  GemvCut best{0, 0};
  double best_t = 1e30;
  for (int64_t nk = 1; nk <= KT && nk <= 64; ++nk) {
    if (nk_only > 0 && nk != nk_only) continue;
    const int64_t tmax = ceil_div(KT, nk);
    if (tmax > act_cap) continue;
    if (tmax * tmt * 4 * kWave > kGFragLoads * kGWaves * kWave || tmax * tmt * 4 > kGWaves * kWave) continue;
    int64_t nbr = 256 / nk;
    if (nbr > nu) nbr = nu;
    if (nbr < 1) break;
    const int64_t umax = ceil_div(nu, nbr);
    if (umax > kGMaxUnits) continue;
    const double stream = (double)umax * tmax * nr * 1152.0 / 25e3;  // us
    const double act = (double)tmax * tmt * kGTileAct / 80e3;
    const double t = (stream + act) + (nk > 1 ? 1.5 : 0.0);
    if (t < best_t) {
      best_t = t;
      best = GemvCut{(int)nbr, (int)nk};
    }
  }
  return best;
}

// Decode kernel use: up to 32 tokens and a cut that fits. By default it is taken where it measured faster than the
// general kernel: with no split k, at least four row units per workgroup (the wide feed-forward projections); with
// a split k, only at up to 16 tokens and where the whole k does not fit in LDS (long rows, such as the feed-forward
// down projection: the general kernel would read the activations from L2 once per wave there). For short rows the
// split-k partial sums cost more memory round trips than the better balance gains.
inline bool gemv_default(const GemvCut& cut, int64_t nu, int64_t KT, int tmt, int nr) {
  if (cut.nbr <= 0) return false;
  // two token tiles halve the k-tiles a workgroup holds in LDS, so every 7B/32B row length takes the split-k form,
  // which measured slower than the general kernel at 17-32 tokens (7B q|k|v 31.8 vs 17.7 us, o 18.5 vs 13.1 us,
  // down 32.0 vs 31.6 us; 32B q|k|v 21.2 vs 17.8 us)
  if (cut.nk > 1 && tmt >= 2) return false;
  if (cut.nk > 1) return KT > gemv_act_cap(tmt, nr);
  return ceil_div(nu, cut.nbr) >= 4;
}

// Options of one call (qn_linear_opts, zero = defaults).
// The caller's event pair of a call's main kernel (both null: none). With a pair the launch goes through
// hipExtLaunchKernel, which records the two events at the launch's own begin and end, the interval a kernel trace
// reports (an event recorded on the stream before and after a launch also takes in its dispatch).
struct MainEvents {
  hipEvent_t begin = nullptr, end = nullptr;
};

struct Opts {
  int kernel = QN_KERNEL_AUTO, nk = 0, depth = 0, rows = 0, waves = 0, elem = 0;
  MainEvents ev;
};

inline bool opts_valid(const Opts& o) {
  return o.kernel >= QN_KERNEL_AUTO && o.kernel <= QN_KERNEL_WIDE && o.nk >= 0 && o.nk <= 64 &&
         (o.depth == 0 || o.depth == 2 || o.depth == 3) && o.rows >= 0 && o.waves >= 0 && (o.rows > 0) == (o.waves > 0) &&
         (o.elem == 0 || o.elem == 1) && (o.ev.begin == nullptr) == (o.ev.end == nullptr);
}

inline Opts opts_of(const qn_linear_opts* p) {
  Opts o;
  if (p) {
    o.kernel = p->kernel;
    o.nk = p->decode_kchunks;
    o.depth = p->decode_depth;
    o.rows = p->general_rows;
    o.waves = p->general_waves;
    o.elem = p->elem_store;
    o.ev.begin = static_cast<hipEvent_t>(p->main_begin);
    o.ev.end = static_cast<hipEvent_t>(p->main_end);
  }
  return o;
}

// Which streaming kernel serves a call: the many-token MFMA kernel, the decode kernel (with its cut) or the general
// kernel. Decided on the host before anything is launched; QN_ERR_UNSUPPORTED if the options name a kernel that
// cannot serve the call.
enum MainPath { kPathGeneral = 0, kPathDecode = 1, kPathMany = 2, kPathFused = 3, kPathWide = 4 };
struct Plan {
  MainPath path = kPathGeneral;
  GemvCut cut{0, 0};
  int depth = 3;
  int ctl_k = 0, nkc = 0, npairs = 0;  // fused decode kernel: LoRA-down items (see FusedArgs)
  bool split = false;  // run as sub-calls of at most kSplitTokens tokens, each with a plan of its own
};
constexpr int64_t kSplitTokens = 64;

// Row blocks x k-chunks of the decode kernel for 17-64 tokens: at most kWSlots units per block, and with a split k
// at most 256 blocks (one arrival counter each). Measured on the 7B shapes at 32-64 tokens, a launch is fastest in one round of workgroups
// (a second round costs about as much as the first, more than the passes it saves) and, within one round, with the
// fewest passes per workgroup; so the cut is the one-round cut with the fewest passes (ties: fewer k-chunks, then
// fewer units per block), else the cut with the fewest rounds x passes. nk_only > 0: that many k-chunks, with the
// fewest units per block that keep one round.
constexpr double kWideMinBytes = 24e6;
inline GemvCut wide_cut(int64_t nu, int64_t KT, int tmt, int nr, int nk_only) {
  (void)tmt;
  (void)nr;
  GemvCut best{0, 0};
  int64_t best_key = INT64_MAX;
  for (int64_t nk = 1; nk <= KT && nk <= 64; ++nk) {
    if (nk_only > 0 && nk != nk_only) continue;
    for (int64_t U = 1; U <= kWSlots; ++U) {
      const int64_t nbr = ceil_div(nu, U);
      if (nk > 1 && nbr > 256) continue;  // (a split k has one arrival counter per block)
      if (nbr > 16384) continue;  // (the kernel forms block * units in 32 bits)
      const int64_t rounds = ceil_div(nbr * nk, 256), passes = ceil_div(ceil_div(KT, nk), kWH);
      const int64_t key = (((rounds > 1 ? 1 : 0) * 4096 + rounds * passes) * 128 + nk) * 8 + U;
      if (key < best_key) {
        best_key = key;
        best = GemvCut{(int)nbr, (int)nk};
      }
    }
  }
  return best;
}

// The fused decode kernel's plan, if it can serve the call: up to 16 tokens, a cut whose chunk fits in LDS beside
// the LoRA-down reduction, with the norm no split k (the row statistics come from the chunk), and LoRA-down items
// (kFItemTiles k-tiles each without a split k; one per chunk with one) that are at most as many as the workgroups.
inline bool plan_fused(int64_t m, int64_t KT, int64_t nu, bool silu, bool norm, const qn_proj* projs,
                       int32_t nproj, int nk_only, Plan* out) {
  if (m < 1 || m > 16 || nu < 1) return false;
  const int nr = silu ? 2 : 1;
  if (norm && nk_only > 1) return false;
  const GemvCut cut = gemv_cut(nu, KT, 1, nr, norm ? 1 : nk_only, (kGLds - fused_lds_top(nr)) / kGTileAct);
  if (cut.nbr <= 0) return false;
  int npairs = 0;
  for (int p = 0; p < nproj; ++p) npairs += (int)ceil_div(projs[p].r, 32);
  const int64_t grid = (int64_t)cut.nbr * cut.nk;
  int64_t nkc = 0, ctl_k = 0;
  if (cut.nk == 1) {
    nkc = ceil_div(KT, kFItemTiles);
    if (npairs > 0 && nkc > grid / npairs) nkc = grid / npairs;
    if (nkc > 64) nkc = 64;
    if (nkc < 1) return false;
    ctl_k = ceil_div(KT, nkc);
    nkc = ceil_div(KT, ctl_k);
  } else {
    nkc = cut.nk;
    if (npairs > cut.nbr) return false;
  }
  if ((int64_t)npairs * nkc > kFMaxItems || (int64_t)npairs * nkc > grid) return false;
  Plan pl;
  pl.path = kPathFused;
  pl.cut = cut;
  pl.ctl_k = (int)ctl_k;
  pl.nkc = (int)nkc;
  pl.npairs = npairs;
  *out = pl;
  return true;
}

// allow_fused: false for a call split into its phases (the fused kernel has no separate prologue). norm: the call
// has the norm (unknown to a workspace query: then the larger of both cases is sized).
inline qn_status plan_main(int64_t m, int64_t KT, int64_t nu, bool silu, bool norm, const qn_proj* projs,
                           int32_t nproj, const Opts& o, bool allow_fused, Plan* out) {
  Plan pl;
  const int nr = silu ? 2 : 1;
  if (o.kernel == QN_KERNEL_FUSED) {
    if (!allow_fused || (o.depth != 0 && o.depth != 3) || !plan_fused(m, KT, nu, silu, norm, projs, nproj, o.nk, &pl))
      return QN_ERR_UNSUPPORTED;
    *out = pl;
    return QN_OK;
  }
  // AUTO at 65-128 tokens: a call whose 64-token parts would run on the decode kernel for 17-64 tokens runs as
  // sub-calls of at most 64 tokens (rows are independent; measured per call, one call on the general kernel vs two:
  // 7B gate|up at 128 tokens 261 vs 89 us, down 95 vs 82; 32B gate|up 456 vs 159, down 239 vs 107). Not for a call
  // split into its phases (the sub-calls share the workspace).
  if (o.kernel == QN_KERNEL_AUTO && allow_fused && m > kSplitTokens && m <= kMaxTokensPerLaunch) {
    Plan sub;
    if (plan_main(kSplitTokens, KT, nu, silu, norm, projs, nproj, o, allow_fused, &sub) == QN_OK &&
        sub.path == kPathWide) {
      pl.path = kPathWide;
      pl.split = true;
      *out = pl;
      return QN_OK;
    }
  }
  // AUTO takes the decode kernel for 17-64 tokens for calls with at least kWideMinBytes of weights (measured on the
  // 7B/32B shapes: the wide feed-forward projections and the long-row down projection run 1.2-1.9x faster than on
  // the general kernel, the 32B gate|up also in the two rounds of workgroups its 1,728 pairs need; smaller
  // projections, such as q|k|v and o, ran as fast or faster on the general kernel)
  bool wide_auto = o.kernel == QN_KERNEL_AUTO && m > 16 && m <= 64 && o.depth != 2 &&
                   (double)nu * KT * nr * 1152.0 >= kWideMinBytes;
  if (wide_auto) wide_auto = wide_cut(nu, KT, m <= 32 ? 2 : 4, nr, o.nk).nbr > 0;
  if (o.kernel == QN_KERNEL_WIDE || wide_auto) {
    if (m <= 16 || m > 64 || (o.depth != 0 && o.depth != 3)) return QN_ERR_UNSUPPORTED;
    pl.path = kPathWide;
    pl.cut = wide_cut(nu, KT, m <= 32 ? 2 : 4, nr, o.nk);
    if (pl.cut.nbr <= 0) return QN_ERR_UNSUPPORTED;
    *out = pl;
    return QN_OK;
  }
  if (o.kernel == QN_KERNEL_MANY || (o.kernel == QN_KERNEL_AUTO && m > kMaxTokensPerLaunch)) {
    if (m <= kMaxTokensPerLaunch) return QN_ERR_UNSUPPORTED;
    pl.path = kPathMany;
  } else if (o.kernel == QN_KERNEL_DECODE || (o.kernel == QN_KERNEL_AUTO && m >= 1 && m <= 32)) {
    bool take = false;
    if (m >= 1 && m <= 32) {
      const int tmt = (int)ceil_div(m, 16);
      pl.cut = gemv_cut(nu, KT, tmt, nr, o.kernel == QN_KERNEL_DECODE ? o.nk : 0, gemv_act_cap(tmt, nr));
      take = o.kernel == QN_KERNEL_DECODE ? pl.cut.nbr > 0 : gemv_default(pl.cut, nu, KT, tmt, nr);
    }
    if (o.kernel == QN_KERNEL_DECODE && !take) return QN_ERR_UNSUPPORTED;
    pl.path = take ? kPathDecode : kPathGeneral;
    pl.depth = o.depth ? o.depth : 3;
  }
  *out = pl;
  return QN_OK;
}

// Split-k part sums of the decode kernel (none without a split).
size_t gemv_pbuf_bytes(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj, const Opts& o) {
  if (!projs || nproj < 1 || m < 1 || m > kMaxTokensPerLaunch) return 0;
  if (m > kSplitTokens) {  // (a call run as sub-calls: the larger of theirs)
    const size_t a = gemv_pbuf_bytes(kSplitTokens, k, projs, nproj, o);
    const size_t b = gemv_pbuf_bytes(m - kSplitTokens, k, projs, nproj, o);
    return a > b ? a : b;
  }
  int tmt = (int)ceil_div(m, 16);
  if (tmt == 3) tmt = 4;  // (the wide decode kernel's token tiles)
  const int64_t KT = ceil_div(k, kKTile);
  int64_t nu_flat = 0;
  for (int p = 0; p < nproj; ++p) nu_flat += ceil_div(projs[p].n, 16);
  // the workspace query does not know the epilogue: size for both readings of a two-projection call
  // nor whether the call is split into phases (no fused kernel then): size for every case
  size_t bytes = 0;
  for (int silu = 0; silu <= (nproj == 2 ? 1 : 0); ++silu)
    for (int fused = 0; fused <= 1; ++fused)
      for (int norm = 0; norm <= 1; ++norm) {
        Plan pl;
        if (plan_main(m, KT, silu ? ceil_div(projs[0].n, 16) : nu_flat, silu, norm != 0, projs, nproj, o, fused != 0,
                      &pl) != QN_OK)
          continue;
        if ((pl.path != kPathDecode && pl.path != kPathFused && pl.path != kPathWide) || pl.cut.nk <= 1) continue;
        const size_t b = (size_t)pl.cut.nbr * (pl.cut.nk + 1) * gemv_block_floats(silu ? 2 : 1, tmt) * 4;
        bytes = b > bytes ? b : bytes;
      }
  return bytes;
}

// ------------------------------------------------------------------------------------------------------------------
// T: LoRA-down sums for the many-token kernel: t of (projection, token tile, 32-rank chunk) = its k-chunk partials
// added in chunk order, split into bf16 hi and lo B-fragments, [p][tile][jc][hi, lo][lane] x 16 bytes. One wave each.
struct TsumArgs {
  const u32x4* t_part;
  u32x4* t_fin;
  int32_t ks, ntiles;
  int32_t r[kMaxProj];
};

__global__ void __launch_bounds__(kWave) k_lora_tsum(TsumArgs a) {
  const int tile = blockIdx.x, p = blockIdx.y, jc = blockIdx.z, lane = threadIdx.x;
  int r = 0;
#pragma unroll
  for (int q = 0; q < kMaxProj; ++q)
    if (q == p) r = a.r[q];
  if (jc * 32 >= r) return;
  const u32x4* src = a.t_part + (((int64_t)(p * a.ntiles + tile) * kRankChunks + jc) * a.ks) * kWave * 2 + lane * 2;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.ks; c0 += 4) {
    u32x4 q[4][2];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = c0 + v < a.ks ? c0 + v : a.ks - 1;
      q[v][0] = gload(src + (int64_t)c * kWave * 2);
      q[v][1] = gload(src + (int64_t)c * kWave * 2 + 1);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (c0 + v < a.ks) {
        s0 += __builtin_bit_cast(f32x4, q[v][0]);
        s1 += __builtin_bit_cast(f32x4, q[v][1]);
      }
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = e < 4 ? s0[e] : s1[e - 4];
    const uint32_t th = f32_to_bf16(t);
    const uint32_t tl = f32_to_bf16(t - bf16_to_f32((uint16_t)th));  // t - th is exact in f32
    if (e % 2 == 0) {
      hi[e / 2] = th;
      lo[e / 2] = tl;
    } else {
      hi[e / 2] |= th << 16;
      lo[e / 2] |= tl << 16;
    }
  }
  u32x4* dst = a.t_fin + (((int64_t)(p * a.ntiles + tile) * kRankChunks + jc) * 2) * kWave + lane;
  dst[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
  dst[kWave] = u32x4{lo[0], lo[1], lo[2], lo[3]};
}

// ------------------------------------------------------------------------------------------------------------------
// M: MFMA kernel for many tokens (prefill / log-prob forward, M > 128). Workgroup tile: 128 tokens (8 token tiles) x
// 32 row groups (512 rows; with SILU 16 (gate, up) pairs); 8 waves, wave w owning row-group slots 4w .. 4w + 3 for
// all 128 tokens, so every weight fragment is loaded and converted once per workgroup. Per k-tile the activation
// fragments of the 128 tokens (32 KB) are loaded straight into LDS, four stages (one LDS array each, loads three
// k-tiles ahead), and read by every wave; each wave loads its own codes and scales into registers, one k-tile
// ahead. The activations of this path carry one power of two per token (the same in every k-tile), so the MFMAs
// accumulate the whole row and the token's 2^-p is applied once, in the epilogue. Workgroups are numbered so that
// those running at the same time on one XCD (one L2) share a few row blocks and token blocks.
constexpr int kMWaves = 8;
constexpr int kMTT = 8;                              // token tiles per workgroup
constexpr int kMRG = 32;                             // row groups per workgroup
constexpr int kMTBGroup = 4;                         // token blocks per group of the workgroup order
constexpr int kMAct = kMTT * 4 * kWave * 16;         // activation fragments per stage (32 KB)
// 16-byte activation loads into LDS per k-tile and wave
constexpr int kMActLoads = 4;

struct GemmArgs {
  LinearArgs L;
  const u32x4* t_fin;       // LoRA t fragments from k_lora_tsum
  const uint32_t* xmx_sc;   // MX weights: the activations' E8M0 words [tile block][k-tile][lane][tile % 8][hi, lo]
  int32_t KT, ntiles, nrg;  // k-tiles; token tiles; row groups (flattened; with SILU: pairs x 2)
  int32_t nrb, ntb;         // row blocks and token blocks of the grid
  int32_t fast_store;       // outputs and residuals allow 16-byte accesses and no output is broadcast
  int32_t t_lds;            // SILU with both ranks <= 32: the LoRA t fragments are staged in LDS for the epilogue
};

struct MW {
  uint32_t c[4][4];  // [row-group slot][32-wide slice]
  uint32_t sc[4];
};

// E2M1 codes (8 per dword) of one 32-wide slice times the E4M3 block scale, exactly, as the f16 A-fragment
__device__ __forceinline__ f16x8 dequant_frag(uint32_t cw, uint32_t scale_byte) {
  const f16x2 sh = __builtin_bit_cast(f16x2, scale_byte * 0x00800080u);  // E4M3 byte << 7 = E4M3 * 2^-8 in f16
  const f16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 0) * sh;
  const f16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 1) * sh;
  const f16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 2) * sh;
  const f16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 3) * sh;
  return f16x8{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
}

// MX: weights in the canonical MXFP4 layout (codes [n][k/2], E8M0 scales [n][k/32]) on the scaled FP4 x FP8 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4: one k-tile per instruction), against activations given as E4M3 hi and lo parts
// with E8M0 block scales (two MFMAs per product, no unpack); no tensor scale and no per-token exponent.
constexpr int kMSc = kWave * 16 * 4;  // activation scale words of a stage: [lane][token tile][hi, lo]
static_assert(kMSc == kMxScStage, "activation scale stage");
struct MWX {
  u32x4 c[4];       // the lane's 32 codes (row lane % 16, 32-block lane / 16) of each slot
  uint32_t sc[4];   // their E8M0 scale
};
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

template <bool SILU, bool MX>
__global__ void __launch_bounds__(kMWaves * kWave) k_gemm(GemmArgs g) {
  // Four stages. Stages 2 and 3 are arrays of their own: the compiler then knows that a stage being read and one
  // being filled by a load into LDS never overlap, and issues no wait for the in-flight fills before each stage's
  // reads (with one array and wave-dependent fill offsets it drained every load before every k-tile). After the loop
  // stages 0 and 1 hold the output tile and stage 3 the LoRA t fragments.
  __shared__ __attribute__((aligned(16))) uint8_t s_st[2 * kMAct];
  __shared__ __attribute__((aligned(16))) uint8_t s_st2a[kMAct];
  __shared__ __attribute__((aligned(16))) uint8_t s_st3a[kMAct];
  uint8_t* const s_st0 = s_st;
  uint8_t* const s_st1 = s_st + kMAct;
  uint8_t* const s_st2 = s_st2a;
  uint8_t* const s_st3 = s_st3a;
  __shared__ __attribute__((aligned(16))) uint8_t s_sc0[MX ? kMSc : 16];  // MX: the stages' activation scales
  __shared__ __attribute__((aligned(16))) uint8_t s_sc1[MX ? kMSc : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_sc2[MX ? kMSc : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_sc3[MX ? kMSc : 16];
  __shared__ ProjEpi s_pe[kMaxProj];
  __shared__ float s_tsc[kMTT * 16];  // the tokens' 2^-p
  const LinearArgs& a = g.L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int KT = g.KT;
  const int kh = (int)(a.k / 2), ks32 = (int)(a.k / 32);  // MX: bytes of codes and of scales per row

  // workgroup -> (row block, token block). Workgroup ids go round-robin over the 8 XCDs; each XCD's ids are given a
  // contiguous range of tiles, walked kMTBGroup token blocks at a time, row blocks outer.
  int rb, tb;
  {
    const int nrb = g.nrb, ntb = g.ntb, nwg = nrb * ntb;
    const int id = blockIdx.x;
    const int x = id % 8, q = nwg / 8, rem = nwg % 8;
    const int gi = x * q + (x < rem ? x : rem) + id / 8;
    const int grp = gi / (kMTBGroup * nrb), idx = gi % (kMTBGroup * nrb);
    const int gsz = ntb - grp * kMTBGroup < kMTBGroup ? ntb - grp * kMTBGroup : kMTBGroup;
    tb = grp * kMTBGroup + idx % gsz;
    rb = idx / gsz;
  }
  const int tile0 = tb * kMTT;
  const int ntl = g.ntiles - tile0 < kMTT ? g.ntiles - tile0 : kMTT;

  // the wave's four row-group slots; slots 2p and 2p + 1 of every wave form epilogue pass p, which covers
  // contiguous rows: SILU slot jj = (pair rb*16 + (jj/2)*8 + wave, projection jj%2); else flattened row group
  // rb*32 + (jj/2)*16 + 2*wave + jj%2
  rsrc_t cd[4], sd[4];
  int pj[4];
  int64_t rgl[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    int p;
    int64_t rl;
    bool live;
    if (SILU) {
      p = jj & 1;
      rl = (int64_t)rb * (kMRG / 2) + (jj / 2) * kMWaves + wave;
      live = rl * 16 < a.p[0].n;
    } else {
      const int64_t gf = (int64_t)rb * kMRG + (jj / 2) * (2 * kMWaves) + 2 * wave + (jj & 1);
      p = 0;
      for (int q = 1; q < a.nproj; ++q)
        if (gf >= a.p[q].rg_begin) p = q;
      p = __builtin_amdgcn_readfirstlane(p);
      rl = gf - a.p[p].rg_begin;
      live = gf < g.nrg && rl * 16 < a.p[p].n;
    }
    pj[jj] = p;
    rgl[jj] = rl;
    const ProjArgs& P = a.p[p];
    if (MX) {  // the row group's rows that exist (the canonical layout has no padding rows)
      const int64_t rows = live ? (P.n - rl * 16 < 16 ? P.n - rl * 16 : 16) : 0;
      cd[jj] = make_rsrc(P.codes + rl * 16 * kh, rows * kh);
      sd[jj] = make_rsrc(P.scales + rl * 16 * ks32, rows * ks32);
    } else {
      cd[jj] = make_rsrc(P.codes + rl * KT * kTileCodeBytes, live ? (int64_t)KT * kTileCodeBytes : 0);
      sd[jj] = make_rsrc(P.scales + rl * KT * kTileScaleBytes, live ? (int64_t)KT * kTileScaleBytes : 0);
    }
  }
  const uint32_t c_off = lane * 16, s_off = ((lane % 16) * 2 + (lane / 16) / 2) * 4;
  const rsrc_t xsrc = make_rsrc(a.xs + (int64_t)tile0 * KT * 4 * kWave, (int64_t)ntl * KT * 4 * kWave * 16);

  // loads of k-tile kt (past KT: out of range, no memory traffic, same instruction count)
  auto act_load = [&](uint8_t* st, int kt) {
    const bool in = kt < KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // first 16-byte piece of this wave (wave masked: a bound the compiler can see, so the fill provably stays
      // inside its stage)
      const int q0 = i * kMWaves * kWave + (wave & (kMWaves - 1)) * kWave;
      const int tt = q0 >> 8, rem = q0 & 255;
      const int so = __builtin_amdgcn_readfirstlane(in ? ((tt * KT + kt) * 4 * kWave + rem) * 16 : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrc, (__attribute__((address_space(3))) void*)(st + q0 * 16), 16,
                                               (in && tt < ntl) ? lane * 16 : kOutOfRange, so, 0, 0);
    }
  };
  // LoRA t fragments of the workgroup's token tiles for both projections (rank chunk 0: hi and lo parts), as
  // 32 pieces of 1 KB [projection][token tile][hi/lo]; four pieces per wave, like one k-tile's activations
  auto t_load = [&](uint8_t* st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = wave * 4 + i, p = q >> 4, tt = (q >> 1) & 7, hl = q & 1;
      const rsrc_t tsrc = make_rsrc(g.t_fin + (int64_t)(p * g.ntiles + tile0) * kRankChunks * 2 * kWave,
                                    (int64_t)ntl * kRankChunks * 2 * kWave * 16);
      const int so = __builtin_amdgcn_readfirstlane((tt * kRankChunks * 2 + hl) * kWave * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(tsrc, (__attribute__((address_space(3))) void*)(st + q * kWave * 16), 16,
                                               tt < ntl ? lane * 16 : kOutOfRange, so, 0, 0);
    }
  };
  // weights of k-tile kt: half h = slices 2h, 2h + 1 of the four slots (8 bytes per lane), or the scales
  auto w_load_half = [&](MW& w, int kt, int h) {
    const bool in = kt < KT;
    const int kc = __builtin_amdgcn_readfirstlane(in ? kt * kTileCodeBytes : 0);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(cd[jj], in ? c_off + 8 * h : kOutOfRange, kc, 0);
      w.c[jj][2 * h] = v[0];
      w.c[jj][2 * h + 1] = v[1];
    }
  };
  auto w_load_sc = [&](MW& w, int kt) {
    const bool in = kt < KT;
    const int ks = __builtin_amdgcn_readfirstlane(in ? kt * kTileScaleBytes : 0);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) w.sc[jj] = __builtin_amdgcn_raw_buffer_load_b32(sd[jj], in ? s_off : kOutOfRange, ks, 0);
  };
  // MX: the lane's codes and scale of k-tile kt for every slot (a 32-block past k, or a tile past KT, reads 0), and
  // the activation scale words of the stage (1 KB per wave pair: every wave issues two 4-byte loads per lane, so the
  // wait counts are the same in every wave)
  auto w_load_mx = [&](MWX& w, int kt) __attribute__((always_inline)) {
    const bool in = kt < KT && kt * kKTile + (lane / 16) * 32 < (int)a.k;
    const uint32_t co = (uint32_t)((lane % 16) * kh + (lane / 16) * 16), so = (uint32_t)((lane % 16) * ks32 + lane / 16);
    const int kc = __builtin_amdgcn_readfirstlane(kt < KT ? kt * 64 : 0), kb = __builtin_amdgcn_readfirstlane(kt < KT ? kt * 4 : 0);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      w.c[jj] = __builtin_amdgcn_raw_buffer_load_b128(cd[jj], in ? co : kOutOfRange, kc, 0);
      w.sc[jj] = __builtin_amdgcn_raw_buffer_load_b8(sd[jj], in ? so : kOutOfRange, kb, 0);
    }
  };
  const rsrc_t scsrc = make_rsrc(g.xmx_sc + (int64_t)(tile0 / kMTT) * KT * (kMSc / 4), MX ? (int64_t)KT * kMSc : 0);
  auto sc_load = [&](uint8_t* scst, int kt) __attribute__((always_inline)) {
    const bool in = kt < KT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q0 = (2 * (wave & (kMWaves - 1)) + i) * kWave * 4;  // this load's first byte in the stage (256 each)
      const int so = __builtin_amdgcn_readfirstlane(in ? kt * kMSc + q0 : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(scsrc, (__attribute__((address_space(3))) void*)(scst + q0), 4,
                                               in ? lane * 4 : kOutOfRange, so, 0, 0);
    }
  };

  f32x4 acc[4][kMTT];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int i = 0; i < kMTT; ++i) acc[jj][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one k-tile: per 32-wide slice, the 8 token tiles' activation fragments from LDS (all eight reads issued
  // first), the wave's four weight fragments unpacked, then 32 MFMAs in groups of four; the weights of the next
  // k-tile are requested as the slices that held them are unpacked
  auto compute = [&](const uint8_t* st, MW& w, int kt_next) {
    const uint8_t* const stl = st + lane * 16;  // (one address per stage; the rest are instruction offsets)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 bq[kMTT];
#pragma unroll
      for (int i = 0; i < kMTT; ++i) bq[i] = *reinterpret_cast<const u32x4*>(stl + (i * 4 + s) * kWave * 16);
      f16x8 wv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) wv[jj] = dequant_frag(w.c[jj][s], (w.sc[jj] >> (8 * s)) & 0xFFu);
      if (s == 1) w_load_half(w, kt_next, 0);
      if (s == 3) {
        w_load_half(w, kt_next, 1);
        w_load_sc(w, kt_next);
      }
#pragma unroll
      for (int i = 0; i < kMTT; ++i) {
        const f16x8 bf = __builtin_bit_cast(f16x8, bq[i]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[jj][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[jj], bf, acc[jj][i], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);  // the unpack
      __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);  // the next k-tile's weight requests
#pragma unroll
      for (int q = 0; q < 8; ++q) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };

  // pipeline, step kt: wait for the wave's own activation loads of kt, barrier (every wave is done with stage
  // (kt + 3) % 4 = (kt - 1) % 4 and every wave's part of stage kt has landed), issue the activations of kt + 3,
  // compute kt (which requests the weights of kt + 1). Loads in order: act 0, act 1, act 2, W 0, then per step
  // act kt+3, W kt+1 (12 loads). Before step kt the loads issued after act kt that may be outstanding are at most
  // act kt+1, W kt-1 (landed: used in step kt-1), act kt+2, W kt, i.e. 32.
  // MX: one k-tile: the next k-tile's weights requested first (into the other register set), the lane's 16 scale
  // words from the stage, then per token tile its hi and lo fragments (32 bytes each) and two scaled MFMAs per slot
  auto compute_mx = [&](const uint8_t* st, const uint8_t* scst, const MWX& w, MWX& wn, int kt_next)
      __attribute__((always_inline)) {
    w_load_mx(wn, kt_next);
    // Per token tile: its hi fragment and block exponents are read one tile ahead (a second register set), its lo
    // fragment right after the previous tile's lo products have been issued, so neither LDS read waits in front of
    // the MFMAs (with both read just before their tile, every tile's reads were exposed: 2.14 -> 2.04 ms per call
    // on the 7B gate|up at 8192 tokens). The exponents come two words per tile, not the stage's sixteen at once.
    const uint8_t* const stl = st + lane * 32;
    const uint8_t* const scl = scst + lane * 64;
    i32x8 hb = *reinterpret_cast<const i32x8*>(stl), lb = *reinterpret_cast<const i32x8*>(stl + 2048);
    u32x2 sc = *reinterpret_cast<const u32x2*>(scl);
#pragma unroll
    for (int i = 0; i < kMTT; ++i) {
      i32x8 hbn = hb;
      u32x2 scn = sc;
      if (i + 1 < kMTT) {
        hbn = *reinterpret_cast<const i32x8*>(stl + ((i + 1) * 2) * 2048);
        scn = *reinterpret_cast<const u32x2*>(scl + (i + 1) * 8);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int shi = (int)sc[0], slo = (int)sc[1];
      // the four slots' hi products, then their lo products: each lo MFMA accumulates onto its slot's hi result,
      // issued four instructions earlier (back to back, every second MFMA would wait for the one before it)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const i32x8 aw = {(int)w.c[jj][0], (int)w.c[jj][1], (int)w.c[jj][2], (int)w.c[jj][3], 0, 0, 0, 0};
        acc[jj][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, hb, acc[jj][i], 4, 0, 0, (int)w.sc[jj], 0, shi);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const i32x8 aw = {(int)w.c[jj][0], (int)w.c[jj][1], (int)w.c[jj][2], (int)w.c[jj][3], 0, 0, 0, 0};
        acc[jj][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, lb, acc[jj][i], 4, 0, 0, (int)w.sc[jj], 0, slo);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < kMTT) lb = *reinterpret_cast<const i32x8*>(stl + ((i + 1) * 2 + 1) * 2048);
      // the MFMAs have no memory effects, so without this statement the compiler sinks them past later steps'
      // barriers and holds (spills) every tile's fragments until then; taking the previous tile's results (complete
      // by now) pins the MFMAs above it without waiting for the ones just issued
      if (i > 0)
        asm volatile("" : "+v"(acc[0][i - 1]), "+v"(acc[1][i - 1]), "+v"(acc[2][i - 1]), "+v"(acc[3][i - 1])::"memory");
      __builtin_amdgcn_sched_barrier(0);
      hb = hbn;
      sc = scn;
    }
    asm volatile("" : "+v"(acc[0][kMTT - 1]), "+v"(acc[1][kMTT - 1]), "+v"(acc[2][kMTT - 1]), "+v"(acc[3][kMTT - 1])::"memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  MW W;
  MWX WX[2];
  if constexpr (MX) {
    act_load(s_st0, 0);
    sc_load(s_sc0, 0);
    act_load(s_st1, 1);
    sc_load(s_sc1, 1);
    act_load(s_st2, 2);
    sc_load(s_sc2, 2);
    w_load_mx(WX[0], 0);
  } else {
    act_load(s_st0, 0);
    act_load(s_st1, 1);
    act_load(s_st2, 2);
    w_load_half(W, 0, 0);
    w_load_half(W, 0, 1);
    w_load_sc(W, 0);
  }
  // the epilogue's per-projection parameters and the tokens' 2^-p, fetched now (their latency overlaps that of the
  // first loads) and kept in LDS
  if (threadIdx.x < kMaxProj) {
#pragma unroll
    for (int q = 0; q < kMaxProj; ++q)
      if (threadIdx.x == q && q < a.nproj) {
        const ProjArgs& P = a.p[q];
        s_pe[q] = ProjEpi{P.y, P.res, P.n, P.ldy, P.ld_res, MX ? 1.0f : gload(P.s_g), P.lambda, P.y_dtype,
                          P.y_repeat, P.head_dim, P.rg_begin, P.r};  // (MX weights carry no tensor scale)
      }
  }
  if (threadIdx.x < kMTT * 16) {
    const int i = threadIdx.x / 16;
    if (MX) s_tsc[threadIdx.x] = 1.0f;  // (the block scales carry the activations' range)
    else s_tsc[threadIdx.x] = i < ntl ? gload(a.xsc + (int64_t)(tile0 + i) * KT * 16 + threadIdx.x % 16) : 0.f;
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  constexpr int kWaitAct = vmcnt_imm(2 * (kMActLoads + 12));
  // MX, step kt: loads in order act+scales kt (6), W kt-2 (8), act+scales kt+1, W kt-1, act+scales kt+2, W kt; the
  // ones after act+scales kt may be outstanding: 3 * 8 + 2 * 6
  constexpr int kWaitMX = vmcnt_imm(3 * 8 + 2 * (kMActLoads + 2));
  // A plain s_barrier (a compiler barrier for memory, no fence): a workgroup fence would also wait for the next
  // stages' loads into LDS, which are meant to stay in flight.
  auto step = [&](const uint8_t* st_use, uint8_t* st_next, int kt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitAct);
    asm volatile("s_barrier" ::: "memory");
    act_load(st_next, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(st_use, W, kt + 1);  // (a k-tile past KT has zero weights and zero activations: adds exactly zero)
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step_mx = [&](const uint8_t* st_use, const uint8_t* sc_use, uint8_t* st_next, uint8_t* sc_next, int kt,
                     const MWX& wc, MWX& wn) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitMX);
    asm volatile("s_barrier" ::: "memory");
    act_load(st_next, kt + 3);
    sc_load(sc_next, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute_mx(st_use, sc_use, wc, wn, kt + 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (MX) {
    for (int kt = 0; kt < KT; kt += 4) {
      step_mx(s_st0, s_sc0, s_st3, s_sc3, kt, WX[0], WX[1]);
      step_mx(s_st1, s_sc1, s_st0, s_sc0, kt + 1, WX[1], WX[0]);
      step_mx(s_st2, s_sc2, s_st1, s_sc1, kt + 2, WX[0], WX[1]);
      step_mx(s_st3, s_sc3, s_st2, s_sc2, kt + 3, WX[1], WX[0]);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < kMTT; ++i) mfma_settle(acc[jj][i]);  // (read by the epilogue past the loop's exit)
  } else {
    for (int kt = 0; kt < KT; kt += 4) {
      step(s_st0, s_st3, kt);
      step(s_st1, s_st0, kt + 1);
      step(s_st2, s_st1, kt + 2);
      step(s_st3, s_st2, kt + 3);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is done with the stages

  // the token's 2^-p (exact), per token tile: D column = token = lane % 16
  float tsc[kMTT];
#pragma unroll
  for (int i = 0; i < kMTT; ++i) tsc[i] = s_tsc[i * 16 + lane % 16];
  // With SILU and both ranks <= 32, the LoRA t fragments go to stage 3 (the output tile takes stages 0 and 1) and
  // the B rows of all four slots are requested with them: one memory round trip for the whole LoRA-up.
  const bool t_lds = SILU && g.t_lds != 0;
  const u32x4* const t_st = reinterpret_cast<const u32x4*>(s_st3);
  uint8_t* const otile_base = s_st;
  u32x4 bfr4[4];
  if (t_lds) {
    t_load(s_st3);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const ProjEpi& E = s_pe[pj[jj]];
      const uint16_t* Bm = nullptr;
#pragma unroll
      for (int q = 0; q < kMaxProj; ++q)
        if (q == pj[jj]) Bm = a.p[q].B;
      const rsrc_t bsrc = make_rsrc(Bm, E.n * E.r * 2);
      const int64_t n = rgl[jj] * 16 + lane % 16;
      const int jr = (lane / 16) * 8;
      if (E.r % 8 == 0) {
        bfr4[jj] = bload16(bsrc, (E.r > 0 && n < E.n && jr < E.r) ? (uint32_t)((n * E.r + jr) * 2) : kOutOfRange);
      } else {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t off = (n * E.r + jr + 2 * e) * 2;
          const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
              bsrc, (n < E.n && jr + 2 * e < E.r) ? (uint32_t)off : kOutOfRange, 0, 0);
          const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
              bsrc, (n < E.n && jr + 2 * e + 1 < E.r) ? (uint32_t)(off + 2) : kOutOfRange, 0, 0);
          wv[e] = lo | (hi << 16);
        }
        bfr4[jj] = u32x4{wv[0], wv[1], wv[2], wv[3]};
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // the staged t fragments have landed
  }

  // LoRA-up and epilogue, two slots at a time (with SILU the gate and up slots of one pair): rows of B (bf16)
  // against the t fragments (hi and lo bf16 parts), then D lane l holds rows 4 (l/16) .. + 3 for token l % 16
  auto epilogue_pair = [&](const int j0) __attribute__((always_inline)) {
    f32x4 la[2][kMTT];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < kMTT; ++i) la[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int jj = j0 + u;
      const ProjEpi& E = s_pe[pj[jj]];
      const int r = E.r;
      if (t_lds) {
        if (r == 0) continue;
#pragma unroll
        for (int i = 0; i < kMTT; ++i) {
          const u32x4 thi = t_st[((pj[jj] * kMTT + i) * 2) * kWave + lane];
          const u32x4 tlo = t_st[((pj[jj] * kMTT + i) * 2 + 1) * kWave + lane];
          la[u][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr4[jj]),
                                                             __builtin_bit_cast(bf16x8, thi), la[u][i], 0, 0, 0);
          la[u][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr4[jj]),
                                                             __builtin_bit_cast(bf16x8, tlo), la[u][i], 0, 0, 0);
        }
        continue;
      }
#pragma unroll
      for (int jc = 0; jc < kRankChunks; ++jc) {
        if (jc * 32 >= r) continue;
        const uint16_t* Bm = nullptr;
#pragma unroll
        for (int q = 0; q < kMaxProj; ++q)
          if (q == pj[jj]) Bm = a.p[q].B;
        const rsrc_t bsrc = make_rsrc(Bm, E.n * r * 2);
        const int64_t n = rgl[jj] * 16 + lane % 16;
        const int jr = jc * 32 + (lane / 16) * 8;
        u32x4 bfr;
        if (r % 8 == 0) {
          bfr = bload16(bsrc, (n < E.n && jr < r) ? (uint32_t)((n * r + jr) * 2) : kOutOfRange);
        } else {
          uint32_t wv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t off = (n * r + jr + 2 * e) * 2;
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
                bsrc, (n < E.n && jr + 2 * e < r) ? (uint32_t)off : kOutOfRange, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
                bsrc, (n < E.n && jr + 2 * e + 1 < r) ? (uint32_t)(off + 2) : kOutOfRange, 0, 0);
            wv[e] = lo | (hi << 16);
          }
          bfr = u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
        const rsrc_t tsrc = make_rsrc(g.t_fin + ((int64_t)(pj[jj] * g.ntiles + tile0) * kRankChunks) * 2 * kWave,
                                      (int64_t)ntl * kRankChunks * 2 * kWave * 16);
#pragma unroll
        for (int i = 0; i < kMTT; ++i) {
          const uint32_t o = (uint32_t)(((i * kRankChunks + jc) * 2 * kWave + lane) * 16);
          const u32x4 thi = bload16(tsrc, i < ntl ? o : kOutOfRange);
          const u32x4 tlo = bload16(tsrc, i < ntl ? o + kWave * 16 : kOutOfRange);
          la[u][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr),
                                                             __builtin_bit_cast(bf16x8, thi), la[u][i], 0, 0, 0);
          la[u][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfr),
                                                             __builtin_bit_cast(bf16x8, tlo), la[u][i], 0, 0, 0);
        }
      }
    }
    // Pass j0 / 2: slots j0 and j0 + 1 of the eight waves cover the output columns [n0, n0 + kC) of one
    // projection (with SILU the product's columns). When the outputs allow 16-byte accesses, the results (before
    // the residual) go to an f32 tile in LDS (16-byte units swizzled by token % 16 against bank conflicts) and are
    // then written row by row, 16 bytes per thread; otherwise each element is stored where it is computed.
    constexpr int kC = SILU ? 16 * kMWaves : 32 * kMWaves;
    const int pass = j0 / 2;
    int pp = 0;
    int64_t n0;
    bool fast = g.fast_store != 0;
    if (SILU) {
      n0 = ((int64_t)rb * (kMRG / 2) + pass * kMWaves) * 16;
    } else {
      const int64_t gf0 = (int64_t)rb * kMRG + pass * (2 * kMWaves);
      int p1 = 0;
      for (int q = 1; q < a.nproj; ++q) {
        if (gf0 >= a.p[q].rg_begin) pp = q;
        if (gf0 + 2 * kMWaves - 1 >= a.p[q].rg_begin) p1 = q;
      }
      n0 = (gf0 - a.p[pp].rg_begin) * 16;
      fast = fast && pp == p1;
    }
    // row tl (a token) of the output tile: the rows fill stages 0 and 1, then stage 2, then stage 3
    auto orow = [&](int tl) __attribute__((always_inline)) -> float* {
      constexpr int kRows01 = 2 * kMAct / (kC * 4), kRowsSt = kMAct / (kC * 4);
      static_assert(kRows01 + 2 * kRowsSt >= kMTT * 16, "output tile rows");
      if (tl < kRows01) return reinterpret_cast<float*>(otile_base) + tl * kC;
      if (tl < kRows01 + kRowsSt) return reinterpret_cast<float*>(s_st2) + (tl - kRows01) * kC;
      return reinterpret_cast<float*>(s_st3) + (tl - kRows01 - kRowsSt) * kC;
    };
#pragma unroll
    for (int u = 0; u < (SILU ? 1 : 2); ++u) {
      const int jj = j0 + u;
      const ProjEpi& E = s_pe[pj[jj]];
      const int cb = SILU ? wave * 16 : (2 * wave + u) * 16;  // the slot's first column in the pass
#pragma unroll
      for (int i = 0; i < kMTT; ++i) {
        const int64_t tok = ((int64_t)tile0 + i) * 16 + lane % 16;
        float o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float out = E.sg * (acc[jj][i][e] * tsc[i]) + E.lambda * la[u][i][e];
          if (SILU) {
            const ProjEpi& F = s_pe[pj[jj + 1]];
            const float up = F.sg * (acc[jj + 1][i][e] * tsc[i]) + F.lambda * la[1][i][e];
            out = out / (1.0f + __expf(-out)) * up;
          }
          o4[e] = out;
        }
        if (fast) {
          const int tl = i * 16 + lane % 16, unit = (cb / 4 + lane / 16) ^ (lane % 16);
          *reinterpret_cast<f32x4*>(orow(tl) + unit * 4) = f32x4{o4[0], o4[1], o4[2], o4[3]};
          continue;
        }
        if (tok >= a.m) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t n = rgl[jj] * 16 + (lane / 16) * 4 + e;
          if (n >= E.n) continue;
          float out = o4[e];
          if (E.res) out += bf16_to_f32(E.res[tok * E.ld_res + n]);
          store_output(E.y, E.y_dtype, tok * E.ldy, n, E.y_repeat, E.head_dim, out);
        }
      }
    }
    if (fast) {
      __syncthreads();
      const ProjEpi& E = s_pe[pp];
      // 16-byte output pieces: 8 bf16 (two tile units) or 4 f32 (one unit); consecutive threads take consecutive
      // pieces of a token row
      auto store_phase = [&](auto f32_tag) __attribute__((always_inline)) {
        constexpr bool F32O = decltype(f32_tag)::value;
        constexpr int kNu = F32O ? 1 : 2, kCnt = 4 * kNu, kPerRow = kC / kCnt;
        constexpr int kIters = kMTT * 16 * kPerRow / (kMWaves * kWave);
        static_assert(kMTT * 16 * kPerRow % (kMWaves * kWave) == 0, "pieces per thread");
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
          const int c = it * kMWaves * kWave + (int)threadIdx.x;
          const int tl = c / kPerRow, pc = c % kPerRow;
          const int64_t tok = (int64_t)tile0 * 16 + tl;
          if (tok >= a.m) continue;
          const int64_t n = n0 + (int64_t)pc * kCnt;
          float v[kCnt];
#pragma unroll
          for (int h = 0; h < kNu; ++h) {
            const f32x4 t4 = *reinterpret_cast<const f32x4*>(orow(tl) + ((pc * kNu + h) ^ (tl % 16)) * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[4 * h + q] = t4[q];
          }
          const bool whole = n + kCnt <= E.n;
          if (E.res) {
            const uint16_t* rp = E.res + tok * E.ld_res + n;
            if (whole && !F32O) {
              const u32x4 r8 = *reinterpret_cast<const u32x4*>(rp);
#pragma unroll
              for (int q = 0; q < kCnt; ++q) v[q] += bf16_to_f32((uint16_t)(r8[q / 2] >> (16 * (q % 2))));
            } else {
#pragma unroll
              for (int q = 0; q < kCnt; ++q)
                if (n + q < E.n) v[q] += bf16_to_f32(rp[q]);
            }
          }
          if (F32O) {
            float* yp = reinterpret_cast<float*>(E.y) + tok * E.ldy + n;
            if (whole) {
              *reinterpret_cast<f32x4*>(yp) = f32x4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
              for (int q = 0; q < kCnt; ++q)
                if (n + q < E.n) yp[q] = v[q];
            }
          } else {
            uint16_t* yp = reinterpret_cast<uint16_t*>(E.y) + tok * E.ldy + n;
            if (whole) {
              u32x4 w8;
#pragma unroll
              for (int q = 0; q < 4; ++q)
                w8[q] = (uint32_t)f32_to_bf16(v[2 * q]) | ((uint32_t)f32_to_bf16(v[2 * q + 1]) << 16);
              *reinterpret_cast<u32x4*>(yp) = w8;
            } else {
#pragma unroll
              for (int q = 0; q < kCnt; ++q)
                if (n + q < E.n) yp[q] = f32_to_bf16(v[q]);
            }
          }
        }
      };
      if (E.y_dtype == QN_F32) store_phase(std::true_type{});
      else store_phase(std::false_type{});
      __syncthreads();
    }
  };
  epilogue_pair(0);
  epilogue_pair(2);
}

// A call's main-kernel launch, with the caller's event pair (MainEvents) when there is one.
template <typename K, typename A>
inline void launch_main(K kernel, dim3 grid, dim3 block, hipStream_t s, const MainEvents& ev, const A& args) {
  if (ev.begin) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.begin, ev.end, 0, args);
  else hipLaunchKernelGGL(kernel, grid, block, 0, s, args);
}

template <int TMT, int R, int W, bool SILU>
void launch_linear(const LinearArgs& a, int64_t nwg, hipStream_t s, const MainEvents& ev) {
  launch_main(k_linear<TMT, R, W, SILU>, dim3((unsigned)nwg), dim3(W * kWave), s, ev, a);
}

// The instantiated (TMT, R, W, SILU) combinations; returns false if the combination is not built. With a null
// `a` it only answers whether the combination is built.
bool dispatch_linear(int tmt, int R, int W, bool silu, const LinearArgs* a, int64_t nwg, hipStream_t s,
                     const MainEvents& ev = MainEvents{}) {
#define QN_CASE(T_, R_, W_, S_)                         \
  if (tmt == T_ && R == R_ && W == W_ && silu == S_) { \
    if (a) launch_linear<T_, R_, W_, S_>(*a, nwg, s, ev); \
    return true;                                       \
  }
  QN_CASE(1, 1, 4, false) QN_CASE(1, 1, 8, false) QN_CASE(1, 1, 16, false)
  QN_CASE(1, 2, 4, false) QN_CASE(1, 2, 8, false) QN_CASE(1, 2, 16, false)
  QN_CASE(1, 4, 4, false) QN_CASE(1, 4, 8, false)
  QN_CASE(1, 2, 4, true) QN_CASE(1, 2, 8, true) QN_CASE(1, 2, 16, true)
  QN_CASE(1, 4, 4, true) QN_CASE(1, 4, 8, true)
  QN_CASE(2, 1, 4, false) QN_CASE(2, 1, 8, false)
  QN_CASE(2, 2, 4, false) QN_CASE(2, 2, 8, false)
  QN_CASE(2, 2, 4, true) QN_CASE(2, 2, 8, true)
  QN_CASE(4, 1, 4, false) QN_CASE(4, 1, 8, false) QN_CASE(4, 2, 4, false)
  QN_CASE(4, 2, 4, true)
  QN_CASE(8, 1, 4, false) QN_CASE(8, 2, 4, true)
#undef QN_CASE
  return false;
}

// Launch shape: R row groups per workgroup (more when many tokens share each activation load, fewer when the
// projection has few row groups) and W waves (enough workgroups x waves to keep every CU streaming).
void pick_shape(int tmt, int64_t mt, bool silu, int64_t nrg, int64_t KT, int* R_out, int* W_out) {
  int R;
  if (tmt == 1) R = mt <= 2 ? (silu ? 2 : 1) : (mt <= 8 ? 2 : 4);
  else if (tmt == 2) R = 2;
  else R = silu ? 2 : 1;
  const int rmin = silu ? 2 : 1;
  const int64_t want_waves = 2048;
  // fewer row groups than workgroups worth having: drop towards one row group (one gate/up pair) per workgroup
  while (R > rmin && ceil_div(nrg, R) * 16 < want_waves) R /= 2;
  // register budget: wider tiles leave room for fewer waves per workgroup
  int wmax = tmt >= 8 ? 4 : (tmt >= 4 ? (R == 1 ? 8 : 4) : (tmt == 2 || R == 4 ? 8 : 16));
  int Rf = R;
  if (tmt == 1 && !silu) {
    // measured at 1-16 tokens on the 7B/8B shapes (q|k|v 4,608 x 3,584; o 3,584 x 3,584; 4,096 x 4,096): one row
    // group per workgroup while the row groups fit one per CU, two beyond; at most eight waves (sixteen leave each
    // wave 1-2 k-tiles and cost 0.5-1.9 us more per call)
    Rf = nrg > 256 ? 2 : 1;
    wmax = 8;
  } else if (tmt == 4 && !silu && nrg > 256) {
    // 33-64 tokens: more row groups than CUs would leave a second, mostly empty round of one-group workgroups;
    // two groups per workgroup keep one round (q|k|v 4,608 x 3,584 at 64 tokens: 23.7 instead of 32.8 us)
    Rf = 2;
    wmax = 4;
  }
  const int64_t nwgf = ceil_div(nrg, Rf);
  int W = 4;
  while (W < wmax && nwgf * W < want_waves && KT >= 2 * W) W *= 2;
  *R_out = Rf;
  *W_out = W;
}

inline bool aligned(const void* p, size_t al) { return ((uintptr_t)p % al) == 0; }

// Launch shape of the general kernel for the launch of `mt` tokens starting at token t0 (tmt token tiles, rounded
// up to a built tile count); false if the options name a shape that is not built.
bool general_shape(int64_t mt, bool silu, int64_t nrg, int64_t KT, const Opts& o, int* tmt_out, int* R, int* W) {
  int tmt = (int)ceil_div(mt, 16);
  tmt = tmt <= 2 ? tmt : (tmt <= 4 ? 4 : 8);
  pick_shape(tmt, mt, silu, nrg, KT, R, W);
  if (o.rows > 0) {
    *R = o.rows;
    *W = o.waves;
  }
  *tmt_out = tmt;
  return dispatch_linear(tmt, *R, *W, silu, nullptr, 0, nullptr);
}

// All host-side validation of a call (nothing is launched on failure); on success the plan of its main kernel.
// mx: weights in the canonical MXFP4 layout for the scaled-MFMA kernel (k % 32 == 0; no tensor scale; byte scales).
qn_status validate_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                          const qn_proj* projs, int32_t nproj, int32_t epilogue, const Opts& o, void* workspace,
                          size_t workspace_bytes, Plan* plan, bool check_workspace, bool mx = false) {
  if (!opts_valid(o)) return QN_ERR_VALUE;
  if (m < 0 || k < 0 || k % (mx ? 32 : 16) != 0) return QN_ERR_SHAPE;
  if (!projs) return QN_ERR_NULL;
  if (nproj < 1) return QN_ERR_SHAPE;
  if (nproj > kMaxProj) return QN_ERR_UNSUPPORTED;
  const int32_t phases = epilogue & (QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY);
  epilogue &= ~(QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY);
  if (phases == (QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY)) return QN_ERR_VALUE;
  if (epilogue != QN_EPI_NONE && epilogue != QN_EPI_SILU_MUL) return QN_ERR_VALUE;
  if (epilogue == QN_EPI_SILU_MUL && (nproj != 2 || projs[0].n != projs[1].n)) return QN_ERR_SHAPE;
  for (int p = 0; p < nproj; ++p) {
    const qn_proj& P = projs[p];
    if (P.n < 0) return QN_ERR_SHAPE;
    if (P.r < 0) return QN_ERR_SHAPE;
    if (P.r > kMaxRank) return QN_ERR_UNSUPPORTED;
    if (P.y_dtype != QN_BF16 && P.y_dtype != QN_F32) return QN_ERR_VALUE;
    if (!std::isfinite(P.lambda)) return QN_ERR_VALUE;
    if (P.y_repeat > 1 && (P.head_dim <= 0 || P.n % P.head_dim != 0)) return QN_ERR_SHAPE;
  }
  if (m == 0 || k == 0) return QN_OK;
  if (!x) return QN_ERR_NULL;
  if (ldx < k) return QN_ERR_SHAPE;
  if (!aligned(x, 2)) return QN_ERR_ALIGN;
  for (int p = 0; p < nproj; ++p) {
    const qn_proj& P = projs[p];
    if (P.n == 0) continue;
    const bool needs_y = !(epilogue == QN_EPI_SILU_MUL && p == 1);
    if (!P.codes || !P.block_scales || (!mx && !P.tensor_scale) || (needs_y && !P.y)) return QN_ERR_NULL;
    if (P.r > 0 && (!P.lora_a || !P.lora_b)) return QN_ERR_NULL;
    const int64_t width = P.y_repeat > 1 ? P.n * P.y_repeat : P.n;
    if (needs_y && P.ldy < width) return QN_ERR_SHAPE;
    if (P.residual && P.ld_res < P.n) return QN_ERR_SHAPE;
    if (!aligned(P.codes, 16) || (!mx && (!aligned(P.block_scales, 4) || !aligned(P.tensor_scale, 4))))
      return QN_ERR_ALIGN;
    if (P.r > 0 && (!aligned(P.lora_a, 16) || !aligned(P.lora_b, 2))) return QN_ERR_ALIGN;
    if (P.r > 0 && P.r % 8 == 0 && !aligned(P.lora_b, 16)) return QN_ERR_ALIGN;
  }
  if (aqn) {
    if (!aqn->gamma) return QN_ERR_NULL;
    if (!(aqn->sigma >= 0.0f) || !std::isfinite(aqn->sigma) || !(aqn->eps >= 0.0f) || !std::isfinite(aqn->eps))
      return QN_ERR_VALUE;
    if (aqn->noise && aqn->noise_ld < 0) return QN_ERR_SHAPE;
    if (aqn->draw && aqn->noise) return QN_ERR_VALUE;  // noise is either read or drawn
    if (aqn->draw && aqn->draw_rows < 0) return QN_ERR_SHAPE;
    if (aqn->noise && aqn->noise_ld > 0 && aqn->noise_ld < k) return QN_ERR_SHAPE;
  }
  if (k > 131072) return QN_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: 16 rows of x or of the noise, the LoRA-down partials and every LoRA-B matrix stay below 2 GiB
  if (ldx >= ((int64_t)1 << 26)) return QN_ERR_UNSUPPORTED;
  if (aqn && aqn->noise && aqn->noise_ld >= ((int64_t)1 << 25)) return QN_ERR_UNSUPPORTED;
  for (int p = 0; p < nproj; ++p)
    if ((int64_t)projs[p].n * projs[p].r * 2 >= ((int64_t)1 << 31)) return QN_ERR_UNSUPPORTED;
  // the main kernel's plan (and, for the general kernel, that every launch's shape is built)
  const bool silu = epilogue == QN_EPI_SILU_MUL;
  const int64_t KT = ceil_div(k, kKTile);
  int64_t rg_total = 0;
  for (int p = 0; p < nproj; ++p) rg_total += ceil_div(projs[p].n, 16);
  const int64_t nrg = silu ? 2 * ceil_div(projs[0].n, 16) : rg_total;
  if (mx) {
    if (o.kernel != QN_KERNEL_AUTO) return QN_ERR_UNSUPPORTED;
    *plan = Plan{};
    plan->path = kPathMany;
  } else {
    const qn_status ps = plan_main(m, KT, silu ? ceil_div(projs[0].n, 16) : rg_total, silu, aqn != nullptr, projs,
                                   nproj, o, phases == 0, plan);
    if (ps != QN_OK) return ps;
  }
  if (plan->path == kPathGeneral && nrg > 0) {
    for (int64_t t0 = 0; t0 < m; t0 += kMaxTokensPerLaunch) {
      const int64_t mt = (m - t0) < kMaxTokensPerLaunch ? (m - t0) : kMaxTokensPerLaunch;
      int tmt, R, W;
      if (!general_shape(mt, silu, nrg, KT, o, &tmt, &R, &W)) return QN_ERR_UNSUPPORTED;
    }
  }
  if (plan->path == kPathMany) {
    const int64_t nrb = silu ? ceil_div(ceil_div(projs[0].n, 16), kMRG / 2) : ceil_div(rg_total, kMRG);
    if (nrb * ceil_div(ceil_div(m, 16), kMTT) >= ((int64_t)1 << 31)) return QN_ERR_UNSUPPORTED;
  }
  if (check_workspace) {
    const Workspace wl = workspace_layout(m, k, projs, nproj, o, mx);
    if (!workspace || workspace_bytes < wl.total) return QN_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QN_ERR_ALIGN;
    if (wl.total - wl.t_part >= ((size_t)1 << 31)) return QN_ERR_UNSUPPORTED;
  }
  return QN_OK;
}

// The launches of a validated call.
// row_base: the row of the caller's call that row 0 of this one is (sub-calls of a split call; it keeps the noise
// draws of every row those of the whole call).
qn_status run_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn, const qn_proj* projs,
                     int32_t nproj, int32_t epilogue, const Opts& o, const Plan& plan, void* workspace,
                     hipStream_t s, int64_t row_base = 0, bool mx = false) {
  if (plan.split) {
    // sub-calls of at most kSplitTokens rows, one after another on the stream (they share the workspace, whose size
    // covers each of theirs): x, outputs, residuals and per-row noise advance by the rows before them
    const bool silu_call = (epilogue & ~(QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY)) == QN_EPI_SILU_MUL;
    int64_t nu = 0;
    for (int p = 0; p < nproj; ++p) nu += ceil_div(projs[p].n, 16);
    if (silu_call) nu = ceil_div(projs[0].n, 16);
    for (int64_t t0 = 0; t0 < m; t0 += kSplitTokens) {
      const int64_t ms = m - t0 < kSplitTokens ? m - t0 : kSplitTokens;
      qn_proj sp[kMaxProj];
      for (int p = 0; p < nproj; ++p) {
        sp[p] = projs[p];
        const int64_t esz = projs[p].y_dtype == QN_F32 ? 4 : 2;
        if (sp[p].y) sp[p].y = static_cast<char*>(sp[p].y) + t0 * sp[p].ldy * esz;
        if (sp[p].residual) sp[p].residual += t0 * sp[p].ld_res;
      }
      qn_aqn sa{};
      if (aqn) {
        sa = *aqn;
        if (sa.noise && sa.noise_ld) sa.noise += t0 * sa.noise_ld;
      }
      Plan sub;
      const qn_status ps = plan_main(ms, ceil_div(k, kKTile), nu, silu_call, aqn != nullptr, sp, nproj, o, true, &sub);
      if (ps != QN_OK || sub.split) return QN_ERR_UNSUPPORTED;  // (not reached: every sub-call has a plan)
      const qn_status st = run_linear(x + t0 * ldx, ms, k, ldx, aqn ? &sa : nullptr, sp, nproj, epilogue, o, sub,
                                      workspace, s, row_base + t0);
      if (st != QN_OK) return st;
    }
    return QN_OK;
  }
  const int32_t phases = epilogue & (QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY);
  epilogue &= ~(QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY);
  const bool run_prologue = phases != QN_RUN_MAIN_ONLY, run_main = phases != QN_RUN_PROLOGUE_ONLY;
  const Workspace wl = workspace_layout(m, k, projs, nproj, o, mx);
  char* ws = static_cast<char*>(workspace);
  const int64_t KT = ceil_div(k, kKTile), kp = KT * kKTile;
  const int64_t ntiles = ceil_div(m, 16);
  u32x4* xs = reinterpret_cast<u32x4*>(ws + wl.xs);
  float* xsc = reinterpret_cast<float*>(ws + wl.xsc);
  float* rstd = reinterpret_cast<float*>(ws + wl.rstd);
  int32_t* tok_p = reinterpret_cast<int32_t*>(ws + wl.tok_p);
  const bool gemm_path = plan.path == kPathMany;
  float* t_part = reinterpret_cast<float*>(ws + wl.t_part);
  const int CT = (int)chunk_tiles(KT);
  const int ks = (int)lora_chunks(k);

  // P (and the statistics kernel for many tokens); the fused decode kernel does this work itself
  if (run_prologue && plan.path != kPathFused) {
    PrologueArgs pa{};
    pa.x = x;
    pa.ldx = ldx;
    pa.m = m;
    pa.k = k;
    pa.KT = KT;
    pa.CT = CT;
    pa.ks = ks;
    pa.has_aqn = aqn ? 1 : 0;
    pa.vec_x = ((uintptr_t)x % 16 == 0) && (ldx % 8 == 0);
    if (aqn) {
      pa.gamma = aqn->gamma;
      pa.noise = aqn->noise;
      pa.noise_ld = aqn->noise ? aqn->noise_ld : 0;
      pa.sigma = aqn->sigma;
      pa.eps = aqn->eps;
      pa.vec_g = (uintptr_t)aqn->gamma % 16 == 0;
      pa.vec_z = aqn->noise && (uintptr_t)aqn->noise % 16 == 0 && pa.noise_ld % 4 == 0;
      pa.draw = QnDraw{aqn->draw ? 1 : 0, aqn->seed, aqn->subseed, aqn->row_offset, aqn->draw_rows, row_base};
    }
    int npg = 0;
    for (int p = 0; p < nproj; ++p) {
      pa.A[p] = projs[p].r > 0 ? projs[p].lora_a : nullptr;
      pa.r[p] = projs[p].r;
      for (int jc = 0; jc * 32 < projs[p].r; ++jc) {
        pa.pg_p[npg] = (int8_t)p;
        pa.pg_jc[npg] = (int8_t)jc;
        ++npg;
      }
    }
    pa.npg = npg;
    pa.nproj = nproj;
    pa.xs = xs;
    pa.xsc = xsc;
    pa.t_part = t_part;
    pa.cnt = reinterpret_cast<uint32_t*>(ws + wl.cnt);
    pa.ncnt = kCountWords;
    // the decode kernel for 17-64 tokens takes t summed (its LoRA wave then needs one memory round trip per item)
    if (plan.path == kPathWide) {
      pa.t_fin = reinterpret_cast<u32x4*>(ws + wl.t_fin);
      pa.t_cnt = reinterpret_cast<uint32_t*>(ws + wl.cnt) + kCountWords;
    }
    // many tokens (and every call of the scaled-MFMA kernel): row statistics in a kernel of their own (rstd with the
    // norm, and one exponent per token, which the scaled-MFMA activations do not use: they carry block scales)
    const bool big = m > kMaxTokensPerLaunch || mx;
    pa.rstd_in = big && aqn ? rstd : nullptr;
    pa.tok_p = big && gemm_path && !mx ? tok_p : nullptr;
    pa.xmx_sc = mx ? reinterpret_cast<uint32_t*>(ws + wl.xmx) : nullptr;
    // with many tokens, two pair groups share a workgroup (h of the chunk is computed once for both)
    pa.pgm = big && norm_threads(k) == 256 ? 2 : 1;
    const int npz = npg > 0 ? (npg + pa.pgm - 1) / pa.pgm : 1;
    // with the norm at decode, each token tile's statistics rows are split over four workgroups (a workgroup
    // reads 4 rows in full instead of 16), or over two or one where four would take more than one round of
    // workgroups (7B q|k|v at 64 tokens: 336 workgroups; the same bits either way)
    pa.tgs = 16;
    if (aqn && !big) {
      const int64_t per_split = ntiles * ks * npz;  // workgroups per token group
      pa.tgs = per_split * 4 <= 256 ? 4 : (per_split * 2 <= 256 ? 8 : 16);
    }
    const dim3 grid((unsigned)(ntiles * (16 / pa.tgs)), (unsigned)ks, (unsigned)npz);
    const dim3 block(kProWaves * kWave);
    const bool vec = pa.vec_x && (!aqn || (pa.vec_g && (!aqn->noise || pa.vec_z)));
#define QN_PRO(NT_, AQN_, PGM_)                                                                    \
  do {                                                                                             \
    if (vec) hipLaunchKernelGGL((k_prologue<NT_, AQN_, true, PGM_>), grid, block, 0, s, pa);    \
    else hipLaunchKernelGGL((k_prologue<NT_, AQN_, false, PGM_>), grid, block, 0, s, pa);       \
  } while (0)
#define QN_STATS(NT_, AQN_)                                                                                   \
  do {                                                                                                        \
    if (vec) hipLaunchKernelGGL((k_rowstats<NT_, AQN_, true>), dim3((unsigned)ntiles), dim3(16 * kWave), 0, s, pa, \
                                rstd, tok_p);                                                                 \
    else hipLaunchKernelGGL((k_rowstats<NT_, AQN_, false>), dim3((unsigned)ntiles), dim3(16 * kWave), 0, s, pa,  \
                            rstd, tok_p);                                                                     \
  } while (0)
    if (!aqn) {
      if (big && !mx) QN_STATS(256, false);  // (without the norm the scaled-MFMA path needs no statistics)
      if (pa.pgm == 2) QN_PRO(256, false, 2);
      else QN_PRO(256, false, 1);
    } else if (norm_threads(k) == 256) {
      if (big) QN_STATS(256, true);
      if (pa.pgm == 2) QN_PRO(256, true, 2);
      else QN_PRO(256, true, 1);
    } else {
      if (big) QN_STATS(1024, true);
      QN_PRO(1024, true, 1);
    }
#undef QN_STATS
#undef QN_PRO
  }

  // L
  LinearArgs la{};
  int32_t rg_total = 0;
  for (int p = 0; p < nproj; ++p) {
    const qn_proj& P = projs[p];
    ProjArgs& A = la.p[p];
    A.codes = P.codes;
    A.scales = P.block_scales;
    A.s_g = P.tensor_scale;
    A.A = P.r > 0 ? P.lora_a : nullptr;
    A.B = P.r > 0 ? P.lora_b : nullptr;
    A.y = P.y;
    A.res = P.residual;
    A.n = P.n;
    A.ldy = P.ldy;
    A.ld_res = P.ld_res;
    A.r = P.r;
    A.y_dtype = P.y_dtype;
    A.y_repeat = P.y_repeat;
    A.head_dim = P.head_dim;
    A.lambda = P.lambda;
    A.rg_begin = rg_total;
    rg_total += (int32_t)ceil_div(P.n, 16);
  }
  la.nproj = nproj;
  la.epilogue = epilogue;
  la.m = m;
  la.k = k;
  la.kp = kp;
  la.xs = xs;
  la.xsc = xsc;
  la.t_part = reinterpret_cast<const u32x4*>(t_part);
  la.t_bytes = (int64_t)(wl.pbuf - wl.t_part);
  la.ks = ks;
  const bool silu = epilogue == QN_EPI_SILU_MUL;
  const int64_t nrg = silu ? 2 * ceil_div(projs[0].n, 16) : rg_total;
  if (nrg == 0 || !run_main) return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
  // many tokens: LoRA t sums, then the MFMA kernel
  if (gemm_path) {
    u32x4* t_fin = reinterpret_cast<u32x4*>(ws + wl.t_fin);
    int max_r = 0;
    for (int p = 0; p < nproj; ++p) max_r = projs[p].r > max_r ? projs[p].r : max_r;
    if (max_r > 0) {
      TsumArgs ta{};
      ta.t_part = reinterpret_cast<const u32x4*>(t_part);
      ta.t_fin = t_fin;
      ta.ks = ks;
      ta.ntiles = (int32_t)ntiles;
      for (int p = 0; p < nproj; ++p) ta.r[p] = projs[p].r;
      hipLaunchKernelGGL(k_lora_tsum, dim3((unsigned)ntiles, (unsigned)nproj, (unsigned)kRankChunks), dim3(kWave), 0,
                         s, ta);
    }
    GemmArgs ga{};
    ga.L = la;
    ga.L.tok0 = 0;
    ga.t_fin = t_fin;
    ga.xmx_sc = mx ? reinterpret_cast<const uint32_t*>(ws + wl.xmx) : nullptr;
    ga.KT = (int32_t)KT;
    ga.ntiles = (int32_t)ntiles;
    ga.nrg = (int32_t)nrg;
    ga.nrb = (int32_t)(silu ? ceil_div(ceil_div(projs[0].n, 16), kMRG / 2) : ceil_div(rg_total, kMRG));
    ga.ntb = (int32_t)ceil_div(ntiles, kMTT);
    // 16-byte output (and residual) accesses through an LDS tile where the buffers allow them and the options do not
    // ask for per-element stores
    bool fast = o.elem == 0;
    for (int p = 0; p < (silu ? 1 : nproj); ++p) {
      const qn_proj& P = projs[p];
      const int64_t esz = P.y_dtype == QN_F32 ? 4 : 2;
      fast = fast && P.y && (uintptr_t)P.y % 16 == 0 && (P.ldy * esz) % 16 == 0 && P.y_repeat <= 1;
      if (P.residual) fast = fast && (uintptr_t)P.residual % 16 == 0 && (P.ld_res * 2) % 16 == 0;
    }
    ga.fast_store = fast ? 1 : 0;
    ga.t_lds = silu && projs[0].r <= 32 && projs[1].r <= 32 ? 1 : 0;
    const dim3 grid((unsigned)(ga.nrb * ga.ntb)), block(kMWaves * kWave);
    if (mx) {
      if (silu) launch_main(k_gemm<true, true>, grid, block, s, o.ev, ga);
      else launch_main(k_gemm<false, true>, grid, block, s, o.ev, ga);
    } else {
      if (silu) launch_main(k_gemm<true, false>, grid, block, s, o.ev, ga);
      else launch_main(k_gemm<false, false>, grid, block, s, o.ev, ga);
    }
    return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
  }
  if (plan.path == kPathFused) {
    FusedArgs fa{};
    GemvArgs& ga = fa.G;
    ga.L = la;
    ga.L.tok0 = 0;
    ga.KT = (int32_t)KT;
    ga.ntiles = 1;
    ga.mt = (int32_t)m;
    ga.nu = (int32_t)(silu ? ceil_div(projs[0].n, 16) : rg_total);
    ga.nbr = plan.cut.nbr;
    ga.nk = plan.cut.nk;
    ga.pbuf = reinterpret_cast<float*>(ws + wl.pbuf);
    ga.cnt = reinterpret_cast<uint32_t*>(ws + wl.cnt);
    fa.x = x;
    fa.ldx = ldx;
    bool vec = ((uintptr_t)x % 16 == 0) && (ldx % 8 == 0);
    if (aqn) {
      fa.gamma = aqn->gamma;
      fa.noise = aqn->noise;
      fa.noise_ld = aqn->noise ? aqn->noise_ld : 0;
      fa.sigma = aqn->sigma;
      fa.eps = aqn->eps;
      fa.draw = QnDraw{aqn->draw ? 1 : 0, aqn->seed, aqn->subseed, aqn->row_offset, aqn->draw_rows, row_base};
      vec = vec && (uintptr_t)aqn->gamma % 16 == 0 &&
            (!aqn->noise || ((uintptr_t)aqn->noise % 16 == 0 && fa.noise_ld % 4 == 0));
      // one gamma + sigma * noise for every token: noise read with a zero stride, one draw for all rows, or none
      fa.g_shared = aqn->draw ? (aqn->draw_rows == 0 || aqn->draw_rows >= m) : (!aqn->noise || fa.noise_ld == 0);
    }
    fa.ctl_k = plan.ctl_k;
    fa.nkc = plan.nkc;
    fa.nitems = plan.npairs * plan.nkc;
    int pair = 0;
    for (int p = 0; p < nproj; ++p) {
      fa.pair0[p] = pair;
      pair += (int)ceil_div(projs[p].r, 32);
    }
    fa.t_part = reinterpret_cast<float*>(ws + wl.t_fused);
    fa.ctl = reinterpret_cast<uint32_t*>(ws + wl.cnt) + 256;
    const dim3 grid((unsigned)(plan.cut.nbr * plan.cut.nk)), block(kGWaves * kWave);
    const bool gsh = aqn && fa.g_shared;
#define QN_FGEMV(S_, A_, V_, G_)                                                                     \
  if (silu == S_ && (aqn != nullptr) == A_ && vec == V_ && gsh == G_) {                             \
    launch_main(k_fgemv<S_, A_, V_, G_>, grid, block, s, o.ev, fa);                                 \
    return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;                                    \
  }
    QN_FGEMV(false, false, false, false) QN_FGEMV(false, false, true, false)
    QN_FGEMV(true, false, false, false) QN_FGEMV(true, false, true, false)
    QN_FGEMV(false, true, false, false) QN_FGEMV(false, true, true, false)
    QN_FGEMV(true, true, false, false) QN_FGEMV(true, true, true, false)
    QN_FGEMV(false, true, false, true) QN_FGEMV(false, true, true, true)
    QN_FGEMV(true, true, false, true) QN_FGEMV(true, true, true, true)
#undef QN_FGEMV
    return QN_ERR_UNSUPPORTED;  // (not reached)
  }
  if (plan.path == kPathWide) {
    const int tmt = m <= 32 ? 2 : 4;
    u32x4* t_fin = reinterpret_cast<u32x4*>(ws + wl.t_fin);  // (summed by the prologue)
    WideArgs wa{};
    GemvArgs& ga = wa.G;
    ga.L = la;
    ga.L.tok0 = 0;
    ga.KT = (int32_t)KT;
    ga.ntiles = (int32_t)ntiles;
    ga.mt = (int32_t)m;
    ga.nu = (int32_t)(silu ? ceil_div(projs[0].n, 16) : rg_total);
    ga.nbr = plan.cut.nbr;
    ga.nk = plan.cut.nk;
    ga.pbuf = reinterpret_cast<float*>(ws + wl.pbuf);
    ga.cnt = reinterpret_cast<uint32_t*>(ws + wl.cnt);
    wa.t_fin = t_fin;
    wa.t_fin_bytes = (int64_t)(wl.pbuf - wl.t_fin);
    const dim3 grid((unsigned)(plan.cut.nbr * plan.cut.nk)), block(kWWaves * kWave);
#define QN_WIDE(T_, S_, L_)                                                          \
  if (tmt == T_ && silu == S_) {                                                    \
    launch_main(k_wgemv<T_, S_, L_>, grid, block, s, o.ev, wa);                    \
    return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;                    \
  }
    QN_WIDE(2, false, 3) QN_WIDE(2, true, 3) QN_WIDE(4, false, 3) QN_WIDE(4, true, 1)
#undef QN_WIDE
    return QN_ERR_UNSUPPORTED;  // (not reached)
  }
  if (plan.path == kPathDecode) {
    const int tmt = (int)ceil_div(m, 16);
    const int64_t nu = silu ? ceil_div(projs[0].n, 16) : rg_total;
    GemvArgs ga{};
    ga.L = la;
    ga.L.tok0 = 0;
    ga.KT = (int32_t)KT;
    ga.ntiles = (int32_t)ceil_div(m, 16);
    ga.mt = (int32_t)m;
    ga.nu = (int32_t)nu;
    ga.nbr = plan.cut.nbr;
    ga.nk = plan.cut.nk;
    ga.pbuf = reinterpret_cast<float*>(ws + wl.pbuf);
    ga.cnt = reinterpret_cast<uint32_t*>(ws + wl.cnt);
    const dim3 grid((unsigned)(plan.cut.nbr * plan.cut.nk)), block(kGWaves * kWave);
    const int depth = plan.depth;  // weight tiles in flight per wave
#define QN_GEMV(T_, S_, D_)                                                            \
  if (tmt == T_ && silu == S_ && depth == D_) {                                       \
    launch_main(k_gemv<T_, S_, D_>, grid, block, s, o.ev, ga);                        \
    return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;                       \
  }
    QN_GEMV(1, false, 2) QN_GEMV(1, false, 3) QN_GEMV(1, true, 2) QN_GEMV(1, true, 3)
    QN_GEMV(2, false, 2) QN_GEMV(2, false, 3) QN_GEMV(2, true, 2) QN_GEMV(2, true, 3)
#undef QN_GEMV
    return QN_ERR_UNSUPPORTED;  // (not reached: every (tmt <= 2, silu, depth 2 or 3) is built)
  }
  for (int64_t t0 = 0; t0 < m; t0 += kMaxTokensPerLaunch) {
    la.tok0 = t0;
    const int64_t mt = (m - t0) < kMaxTokensPerLaunch ? (m - t0) : kMaxTokensPerLaunch;
    int tmt, R, W;
    general_shape(mt, silu, nrg, KT, o, &tmt, &R, &W);  // (built: checked in validation)
    dispatch_linear(tmt, R, W, silu, &la, ceil_div(nrg, R), s, o.ev);
  }
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

}  // namespace
}  // namespace qn

using namespace qn;

extern "C" size_t nvfp4_lora_linear_workspace_opts(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj,
                                                   const qn_linear_opts* opts) {
  if (m <= 0 || k <= 0 || nproj <= 0 || !projs) return 0;
  const Opts o = opts_of(opts);
  if (!opts_valid(o)) return 0;
  return workspace_layout(m, k, projs, nproj, o).total;
}

extern "C" size_t nvfp4_lora_linear_workspace(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj) {
  return nvfp4_lora_linear_workspace_opts(m, k, projs, nproj, nullptr);
}

extern "C" qn_status nvfp4_lora_linear_opts(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                                            const qn_proj* projs, int32_t nproj, int32_t epilogue,
                                            const qn_linear_opts* opts, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  const Opts o = opts_of(opts);
  Plan plan;
  const qn_status st =
      validate_linear(x, m, k, ldx, aqn, projs, nproj, epilogue, o, workspace, workspace_bytes, &plan, true);
  if (st != QN_OK || m == 0 || k == 0) return st;
  return run_linear(x, m, k, ldx, aqn, projs, nproj, epilogue, o, plan, workspace, (hipStream_t)stream);
}

// ---- the entry point that allocates nothing ---------------------------------------------------------------------
// Its scratch space is one file-scope device array per GPU, held until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): the device address of each GPU's copy is looked
// up once per device with hipGetSymbolAddress and used instead.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's copy of the scratch array (looked up on its first use on that device, with it current).
static qn_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return QN_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QN_OK;
}

extern "C" size_t nvfp4_lora_linear_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" qn_status nvfp4_lora_linear_noalloc(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                                               const qn_proj* projs, int32_t nproj, int32_t epilogue, void* stream) {
  Plan plan;
  const Opts o;
  qn_status st = validate_linear(x, m, k, ldx, aqn, projs, nproj, epilogue, o, nullptr, 0, &plan, false);
  if (st != QN_OK || m == 0 || k == 0) return st;
  if (workspace_layout(m, k, projs, nproj, o).total > kScratchBytes) return QN_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != QN_OK) return st;
  return run_linear(x, m, k, ldx, aqn, projs, nproj, epilogue, o, plan, ws, (hipStream_t)stream);
}

extern "C" size_t mxfp4_lora_linear_workspace(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj) {
  if (m <= 0 || k <= 0 || nproj <= 0 || !projs) return 0;
  return workspace_layout(m, k, projs, nproj, Opts{}, true).total;
}

extern "C" qn_status mxfp4_lora_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                                       const qn_proj* projs, int32_t nproj, int32_t epilogue, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const Opts o;
  Plan plan;
  const qn_status st =
      validate_linear(x, m, k, ldx, aqn, projs, nproj, epilogue, o, workspace, workspace_bytes, &plan, true, true);
  if (st != QN_OK || m == 0 || k == 0) return st;
  return run_linear(x, m, k, ldx, aqn, projs, nproj, epilogue, o, plan, workspace, (hipStream_t)stream, 0, true);
}

extern "C" qn_status nvfp4_lora_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                                       const qn_proj* projs, int32_t nproj, int32_t epilogue, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return nvfp4_lora_linear_opts(x, m, k, ldx, aqn, projs, nproj, epilogue, nullptr, workspace, workspace_bytes,
                                stream);
}

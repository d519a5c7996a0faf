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
constexpr int kRstdKernelTiles = 16;        // token tiles from which the statistics get a kernel of their own

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
  size_t xs, xsc, rstd, t_part, total;
};

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

Workspace workspace_layout(int64_t m, int64_t k, int32_t nproj) {
  const int64_t KT = ceil_div(k, kKTile), kp = KT * kKTile;
  const int64_t mp = ceil_div(m, 16) * 16;
  Workspace w;
  size_t off = 0;
  w.xs = off;     off = align256(off + (size_t)mp * kp * 2);
  w.xsc = off;    off = align256(off + (size_t)mp * KT * 4);
  w.rstd = off;   off = align256(off + (size_t)mp * 4);
  w.t_part = off; off = align256(off + (size_t)nproj * (mp / 16) * kRankChunks * lora_chunks(k) * kWave * 32);
  w.total = off;
  return w;
}

// Loads. Every load issued ahead of the weight stream is a buffer load or a global-segment load, never a flat one:
// a pending flat load may be an LDS access, which forces the compiler to drain all loads at every later wait and
// so would serialize the double-buffered stream.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format (gfx9 family)
constexpr int kNonTemporal = 2;                 // streamed once: do not keep in cache
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past every num_records: the load returns 0

// Wave-uniform copies (readfirstlane) of values the compiler cannot prove uniform on its own, so that buffer
// descriptors built from them stay in SGPRs.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Raw buffer descriptor over [base, base + bytes); bytes < 2^31 (checked on the host).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)uniform64((uint64_t)base), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes), kRsrcWord3);
}

__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Load through a pointer known to address global memory.
template <class T>
__device__ __forceinline__ T gload(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) T*>(reinterpret_cast<uintptr_t>(p));
}

// ------------------------------------------------------------------------------------------------------------------
// Statistics kernel (many tokens): one wave per token, rstd[tok] = 1 / sqrt(mean x^2 + eps).
template <int NT>
__global__ void __launch_bounds__(16 * kWave) k_rstd(const uint16_t* __restrict__ x, int64_t ldx, int64_t m,
                                                     int64_t k, int vec_x, float eps, float* __restrict__ rstd) {
  const int64_t tok = (int64_t)blockIdx.x * 16 + threadIdx.x / kWave;
  if (tok >= m) return;
  const float r = rms_rstd(row_sumsq_one_wave<NT>(x + tok * ldx, k, vec_x != 0), k, eps);
  if (threadIdx.x % kWave == 0) rstd[tok] = r;
}

// ------------------------------------------------------------------------------------------------------------------
// P: prologue. Workgroup (token tile, k-chunk c of CT k-tiles, pair group pg = one 32-rank chunk jc of projection p);
// 16 waves. Every pair group of a chunk computes the same h; pair group 0 stores the MFMA fragments and tile scales.
constexpr int kProWaves = 16;

struct PrologueArgs {
  const uint16_t* x;
  int64_t ldx, m, k, KT;
  int32_t CT, ks, npg, has_aqn;
  int32_t vec_x, vec_g, vec_z;
  const uint16_t* gamma;
  const float* noise;
  int64_t noise_ld;
  float sigma, eps;
  const float* rstd_in;  // statistics from k_rstd, or null: computed here
  const uint16_t* A[kMaxProj];
  int32_t r[kMaxProj];
  int8_t pg_p[kMaxPg], pg_jc[kMaxPg];
  u32x4* xs;
  float* xsc;
  float* t_part;
};

template <int NT, bool AQN>
__global__ void __launch_bounds__(kProWaves * kWave) k_prologue(PrologueArgs a) {
  constexpr int kCT = kMaxChunkTiles;                              // k-tiles per chunk (at most)
  constexpr int kProSlices = kCT * 4 / kProWaves;                // 32-wide k-slices per wave (at most)
  constexpr int kPasses = kCT * 256 / (kProWaves * kWave);        // 8-element groups per thread (at most)
  constexpr int kHRow = kMaxChunkTiles * kKTile + 8;  // LDS row of h (bf16), padded against bank conflicts
  __shared__ float s_rstd[16];
  __shared__ __attribute__((aligned(16))) uint16_t s_h[16][kHRow];
  __shared__ f32x4 s_red[kProWaves][2][kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int64_t tile = blockIdx.x, ntiles = gridDim.x;
  const int c = blockIdx.y, pg = blockIdx.z;
  const int64_t kt0 = (int64_t)c * a.CT;
  const int ctn = (int)(a.KT - kt0 < a.CT ? a.KT - kt0 : a.CT);  // k-tiles in this chunk
  const int64_t kc0 = kt0 * kKTile;
  const bool lora = pg < a.npg;
  const int p = lora ? a.pg_p[pg] : 0, jc = lora ? a.pg_jc[pg] : 0;

  // LoRA-down A fragments of this wave's slices, issued first (they do not depend on x). Fragment (g, slice s): ranks
  // jc*32 + g*16 + lane%16, k = kc0 + 32 s + 8 (lane/16) .. + 8; ranks past r and k past the row read as 0.
  const int nsl = ctn * 4;
  u32x4 af[2][kProSlices];
  if (lora) {
    const int r = a.r[p];
    const rsrc_t asrc = make_rsrc(a.A[p], (int64_t)r * a.k * 2);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < kProSlices; ++i) {
        const int s = wave + i * kProWaves;
        const int j = jc * 32 + g * 16 + lane % 16;
        const int64_t kk = kc0 + (int64_t)s * 32 + (lane / 16) * 8;
        const bool ok = s < nsl && j < r && kk < a.k;
        af[g][i] = bload16(asrc, ok ? (uint32_t)(((int64_t)j * a.k + kk) * 2) : kOutOfRange);
      }
  }

  // inputs of h for this thread's 8-element groups (x, and gamma and noise with the norm), fetched before the
  // statistics so that every load of the prologue is in flight at once. Group g: token g / (ctn*16), k-tile
  // (g % (ctn*16)) / 16 of the chunk; the 16 groups of one (token, k-tile) are 16 consecutive lanes.
  const int ngroups = 16 * ctn * 16;  // a multiple of 256: a wave is either wholly in range or wholly out
  uint32_t hx[kPasses][4], hg[kPasses][4];
  float hz[kPasses][8];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int g = threadIdx.x + ps * kProWaves * kWave;
    const int t = g / (ctn * 16), kg = g % (ctn * 16);
    const int64_t tok = tile * 16 + t, kk = kc0 + (int64_t)kg * 8;
    const bool ok = g < ngroups && tok < a.m && kk < a.k;
#pragma unroll
    for (int e = 0; e < 4; ++e) hx[ps][e] = hg[ps][e] = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) hz[ps][e] = 0.f;
    if (!ok) continue;
    const uint16_t* xr = a.x + tok * a.ldx + kk;
    if (a.vec_x) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(xr);
      hx[ps][0] = q[0]; hx[ps][1] = q[1]; hx[ps][2] = q[2]; hx[ps][3] = q[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) hx[ps][e] = (uint32_t)xr[2 * e] | ((uint32_t)xr[2 * e + 1] << 16);
    }
    if (AQN) {
      if (a.vec_g) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(a.gamma + kk);
        hg[ps][0] = q[0]; hg[ps][1] = q[1]; hg[ps][2] = q[2]; hg[ps][3] = q[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hg[ps][e] = (uint32_t)a.gamma[kk + 2 * e] | ((uint32_t)a.gamma[kk + 2 * e + 1] << 16);
      }
      const float* nz = a.noise ? a.noise + tok * a.noise_ld + kk : nullptr;
      if (nz && a.vec_z) {
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(nz), z1 = *reinterpret_cast<const f32x4*>(nz + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { hz[ps][e] = z0[e]; hz[ps][4 + e] = z1[e]; }
      } else if (nz) {
#pragma unroll
        for (int e = 0; e < 8; ++e) hz[ps][e] = nz[e];
      }
    }
  }

  // statistics: wave w <-> token w of the tile
  if (AQN) {
    const int64_t tok = tile * 16 + wave;
    float rstd = 0.f;
    if (tok < a.m)
      rstd = a.rstd_in ? gload(a.rstd_in + tok)
                       : rms_rstd(row_sumsq_one_wave<NT>(a.x + tok * a.ldx, a.k, a.vec_x != 0), a.k, a.eps);
    if (lane == 0) s_rstd[wave] = rstd;
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
    if (pg == 0) {
      // tile amax over the 16 lanes of this (token, k-tile), then 2^p with amax * 2^p in [2^14, 2^15), read off the
      // exponent field and kept within the normal range so 2^p and 2^-p are plain f32 powers of two
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(hv[e])), fabsf(hi_bf16(hv[e]))));
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
      int pw = 0;
      if (amax > 0.0f) {
        const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127;
        pw = 14 - (e < -126 ? -126 : e);
        pw = pw > 126 ? 126 : pw;
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
      a.xs[((tile * a.KT + kt) * 4 + s) * kWave + lhi * 16 + t] = u32x4{packed[0], packed[1], packed[2], packed[3]};
      if (jj == 0) a.xsc[(tile * a.KT + kt) * 16 + t] = __uint_as_float((uint32_t)(127 - pw) << 23);
    }
  }
  __syncthreads();
  if (!lora) return;

  // LoRA-down over the chunk: B-fragment (token lane%16, k = 32 s + 8 (lane/16) .. + 8) from LDS
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < kProSlices; ++i) {
    const int s = wave + i * kProWaves;
    if (s >= nsl) break;
    const u32x4 b = *reinterpret_cast<const u32x4*>(&s_h[lane % 16][s * 32 + (lane / 16) * 8]);
#pragma unroll
    for (int g = 0; g < 2; ++g)
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[g][i]),
                                                       __builtin_bit_cast(bf16x8, b), acc[g], 0, 0, 0);
  }
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
    a.t_part[((((int64_t)p * ntiles + tile) * kRankChunks + jc) * a.ks + c) * kWave * 8 + L * 8 + jl % 8] = v;
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
        for (int u = 0; u < 8; ++u) {
          if (c0 + u >= a.ks) break;
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
    const int rep = O.y_repeat > 1 ? O.y_repeat : 1;
    for (int g = 0; g < rep; ++g) {
      const int64_t col_out = rep > 1 ? ((n / O.head_dim) * rep + g) * O.head_dim + n % O.head_dim : n;
      const int64_t off = gtok * O.ldy + col_out;
      if (O.y_dtype == QN_F32) reinterpret_cast<float*>(O.y)[off] = out;
      else reinterpret_cast<uint16_t*>(O.y)[off] = f32_to_bf16(out);
    }
  }
}

template <int TMT, int R, int W, bool SILU>
void launch_linear(const LinearArgs& a, int64_t nwg, hipStream_t s) {
  hipLaunchKernelGGL((k_linear<TMT, R, W, SILU>), dim3((unsigned)nwg), dim3(W * kWave), 0, s, a);
}

// The instantiated (TMT, R, W, SILU) combinations; returns false if the combination is not built.
bool dispatch_linear(int tmt, int R, int W, bool silu, const LinearArgs& a, int64_t nwg, hipStream_t s) {
#define QN_CASE(T_, R_, W_, S_)                         \
  if (tmt == T_ && R == R_ && W == W_ && silu == S_) { \
    launch_linear<T_, R_, W_, S_>(a, nwg, s);          \
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
  const int64_t nwg = ceil_div(nrg, R);
  // register budget: wider tiles leave room for fewer waves per workgroup
  const int wmax = tmt >= 8 ? 4 : (tmt >= 4 ? (R == 1 ? 8 : 4) : (tmt == 2 || R == 4 ? 8 : 16));
  int W = 4;
  while (W < wmax && nwg * W < want_waves && KT >= 2 * W) W *= 2;
  *R_out = R;
  *W_out = W;
}

inline bool aligned(const void* p, size_t al) { return ((uintptr_t)p % al) == 0; }

}  // namespace
}  // namespace qn

using namespace qn;

extern "C" size_t nvfp4_lora_linear_workspace(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj) {
  (void)projs;
  if (m <= 0 || k <= 0 || nproj <= 0) return 0;
  return workspace_layout(m, k, nproj).total;
}

extern "C" qn_status nvfp4_lora_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                                       const qn_proj* projs, int32_t nproj, int32_t epilogue, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  // ---- host-side validation (nothing is launched on failure)
  if (m < 0 || k < 0 || k % 16 != 0) return QN_ERR_SHAPE;
  if (!projs) return QN_ERR_NULL;
  if (nproj < 1) return QN_ERR_SHAPE;
  if (nproj > kMaxProj) return QN_ERR_UNSUPPORTED;
  const int32_t phases = epilogue & (QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY);
  epilogue &= ~(QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY);
  if (phases == (QN_RUN_PROLOGUE_ONLY | QN_RUN_MAIN_ONLY)) return QN_ERR_VALUE;
  const bool run_prologue = phases != QN_RUN_MAIN_ONLY, run_main = phases != QN_RUN_PROLOGUE_ONLY;
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
    if (!P.codes || !P.block_scales || !P.tensor_scale || (needs_y && !P.y)) return QN_ERR_NULL;
    if (P.r > 0 && (!P.lora_a || !P.lora_b)) return QN_ERR_NULL;
    const int64_t width = P.y_repeat > 1 ? P.n * P.y_repeat : P.n;
    if (needs_y && P.ldy < width) return QN_ERR_SHAPE;
    if (P.residual && P.ld_res < P.n) return QN_ERR_SHAPE;
    if (!aligned(P.codes, 16) || !aligned(P.block_scales, 4) || !aligned(P.tensor_scale, 4)) return QN_ERR_ALIGN;
    if (P.r > 0 && (!aligned(P.lora_a, 16) || !aligned(P.lora_b, 2))) return QN_ERR_ALIGN;
    if (P.r > 0 && P.r % 8 == 0 && !aligned(P.lora_b, 16)) return QN_ERR_ALIGN;
  }
  if (aqn) {
    if (!aqn->gamma) return QN_ERR_NULL;
    if (!(aqn->sigma >= 0.0f) || !std::isfinite(aqn->sigma) || !(aqn->eps >= 0.0f) || !std::isfinite(aqn->eps))
      return QN_ERR_VALUE;
    if (aqn->noise && aqn->noise_ld < 0) return QN_ERR_SHAPE;
    if (aqn->noise && aqn->noise_ld > 0 && aqn->noise_ld < k) return QN_ERR_SHAPE;
  }
  const Workspace wl = workspace_layout(m, k, nproj);
  if (!workspace || workspace_bytes < wl.total) return QN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return QN_ERR_ALIGN;
  if (k > 131072) return QN_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: the LoRA-down partials and every LoRA-B matrix stay below 2 GiB
  if (wl.total - wl.t_part >= ((size_t)1 << 31)) return QN_ERR_UNSUPPORTED;
  for (int p = 0; p < nproj; ++p)
    if ((int64_t)projs[p].n * projs[p].r * 2 >= ((int64_t)1 << 31)) return QN_ERR_UNSUPPORTED;

  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  const int64_t KT = ceil_div(k, kKTile), kp = KT * kKTile;
  const int64_t ntiles = ceil_div(m, 16);
  u32x4* xs = reinterpret_cast<u32x4*>(ws + wl.xs);
  float* xsc = reinterpret_cast<float*>(ws + wl.xsc);
  float* rstd = reinterpret_cast<float*>(ws + wl.rstd);
  float* t_part = reinterpret_cast<float*>(ws + wl.t_part);
  const int CT = (int)chunk_tiles(KT);
  const int ks = (int)lora_chunks(k);

  // P (and the statistics kernel for many tokens)
  if (run_prologue) {
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
    pa.xs = xs;
    pa.xsc = xsc;
    pa.t_part = t_part;
    const bool big = aqn && ntiles >= kRstdKernelTiles;
    pa.rstd_in = big ? rstd : nullptr;
    const dim3 grid((unsigned)ntiles, (unsigned)ks, (unsigned)(npg > 0 ? npg : 1));
    const dim3 block(kProWaves * kWave);
    if (!aqn) {
      hipLaunchKernelGGL((k_prologue<256, false>), grid, block, 0, s, pa);
    } else if (norm_threads(k) == 256) {
      if (big) hipLaunchKernelGGL(k_rstd<256>, dim3((unsigned)ntiles), block, 0, s, x, ldx, m, k, pa.vec_x, pa.eps, rstd);
      hipLaunchKernelGGL((k_prologue<256, true>), grid, block, 0, s, pa);
    } else {
      if (big) hipLaunchKernelGGL(k_rstd<1024>, dim3((unsigned)ntiles), block, 0, s, x, ldx, m, k, pa.vec_x, pa.eps, rstd);
      hipLaunchKernelGGL((k_prologue<1024, true>), grid, block, 0, s, pa);
    }
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
  la.t_bytes = (int64_t)(wl.total - wl.t_part);
  la.ks = ks;
  const bool silu = epilogue == QN_EPI_SILU_MUL;
  const int64_t nrg = silu ? 2 * ceil_div(projs[0].n, 16) : rg_total;
  if (nrg == 0 || !run_main) return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
  for (int64_t t0 = 0; t0 < m; t0 += kMaxTokensPerLaunch) {
    la.tok0 = t0;
    const int64_t mt = (m - t0) < kMaxTokensPerLaunch ? (m - t0) : kMaxTokensPerLaunch;
    int tmt = (int)ceil_div(mt, 16);
    tmt = tmt <= 2 ? tmt : (tmt <= 4 ? 4 : 8);
    int R, W;
    pick_shape(tmt, mt, silu, nrg, KT, &R, &W);
    // tuning override "R,W" (row groups and waves per workgroup); ignored unless that kernel variant is built
    if (const char* ov = std::getenv("QN_LINEAR_SHAPE")) {
      int r2 = 0, w2 = 0;
      if (std::sscanf(ov, "%d,%d", &r2, &w2) == 2 && r2 > 0 && w2 > 0 && (!silu || r2 % 2 == 0)) {
        R = r2;
        W = w2;
      }
    }
    const int64_t nwg = ceil_div(nrg, R);
    if (!dispatch_linear(tmt, R, W, silu, la, nwg, s)) return QN_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

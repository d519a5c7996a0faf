// The rollout-decode linear layer: y_p = s_g,p * W_hat_p h + lambda_p * B_p (A_p h), h = AQN-RMSNorm(x).
//
// "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops" (technical review):
//   §2.1 forward map y = W_hat x + lambda B (A x) with a frozen quantized base and trainable A, B;
//   §3.1 W_hat = s_g * s_b * q (NVFP4); §3.2 decode reads large packed weights for few tokens, so unpack, scale
//   and conversion must keep up with the byte stream; §5.1 AQN-RMSNorm feeds the projections that share its input.
//
// Three kernels per call, all on the caller's stream:
//   P1 k_norm_convert  one workgroup per token: RMSNorm statistics, h = bf16(x * rstd * (gamma + sigma * noise)) (or
//                      h = x), written row-major for the LoRA branch, plus the MFMA B-fragments of h as f16 scaled by a
//                      per-token power of two 2^p (exact: bf16 has 8 significant bits, f16 11, and the scale keeps the
//                      token's largest magnitude in [2^14, 2^15), so every element above 2^-32 of it converts exactly).
//   P2 k_lora_down     t = A h with bf16 16x16x32 MFMAs over at most 8 k-chunks per projection and token tile; each
//                      chunk's partial sums are stored in the layout of the LoRA-up MFMA's B-fragments.
//   L  k_linear        streams the tiled NVFP4 weight once: per lane one 16-byte load of codes (32 weights) and one
//                      dword of block scales per 128-wide k-tile; FP4 -> f16 with the hardware converter (scale 2^8),
//                      times the E4M3 scale reinterpreted as f16 (byte << 7 is the E4M3 value * 2^-8, exact for
//                      normals and subnormals) gives s_b * q exactly in f16; f16 16x16x32 MFMAs accumulate in f32.
//                      Waves split k; partials meet in LDS. The LoRA term: the chunk partials of t are summed in a fixed
//                      order (so results do not depend on scheduling) and split t = t_hi + t_lo, both bf16 (t - t_hi is
//                      exact in f32, 16 significant bits kept); B t is then two bf16 MFMAs per row group. The epilogue applies s_g, the per-token 2^-p, lambda, residual, SiLU(gate) * up,
//                      broadcast and rounding. Everything the epilogue reads is fetched before the weight stream.
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
constexpr int kMaxTokensPerLaunch = 128;

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
  const float* xunscale;   // [m] 2^-p per token
  const u32x4* t_part;     // LoRA-down partials, [nproj][tile][kRankChunks][ks][64 lanes][8 f32]
  int64_t t_bytes;
  int32_t ks;              // LoRA-down k-chunks
};

// Workspace carve-up (256-byte aligned regions).
struct Workspace {
  size_t xs, xunscale, h, t_part, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// LoRA-down k-chunks: as few as possible, each a multiple of 32 and at most 4096 wide (one pass of the 16 waves)
inline int64_t lora_chunks(int64_t k) { return ceil_div(k, 4096); }
inline int64_t lora_chunk_width(int64_t k) { return ceil_div(ceil_div(k, lora_chunks(k)), 32) * 32; }

Workspace workspace_layout(int64_t m, int64_t k, int32_t nproj) {
  const int64_t kp = ceil_div(k, kKTile) * kKTile;
  const int64_t mp = ceil_div(m, 16) * 16;
  Workspace w;
  size_t off = 0;
  w.xs = off;       off = align256(off + (size_t)mp * kp * 2);
  w.xunscale = off; off = align256(off + (size_t)mp * 4);
  w.h = off;        off = align256(off + (size_t)mp * kp * 2);
  w.t_part = off;   off = align256(off + (size_t)nproj * (mp / 16) * kRankChunks * lora_chunks(k) * kWave * 32);
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
// P1: one workgroup per token row. The row stays in registers between passes: sum of squares -> AQN -> token amax ->
// stores of h (row-major bf16, for the LoRA branch) and of the f16 MFMA B-fragments scaled by 2^p.
template <int NT, int CPT>
__global__ void __launch_bounds__(NT) k_norm_convert(const uint16_t* __restrict__ x, int64_t ldx, int64_t k,
                                                     int64_t kp, int has_aqn, const uint16_t* gamma, const float* noise,
                                                     int64_t noise_ld, float sigma, float eps, int vec_in, int vec_g,
                                                     int vec_z, uint16_t* __restrict__ h_out, u32x4* __restrict__ xs,
                                                     float* __restrict__ xunscale) {
  __shared__ float red[NT / kWave];
  const int64_t row = blockIdx.x;
  RowRegs<CPT> r;
  load_row<NT, CPT>(x + row * ldx, k, vec_in != 0, r);
  if (has_aqn) {
    ScaleRegs<CPT> sr;
    load_scales<NT, CPT>(gamma, noise ? noise + row * noise_ld : nullptr, k, vec_g != 0, vec_z != 0, sr);
    const float rstd = rms_rstd(row_sumsq<NT, CPT>(r, red), k, eps);
    apply_aqn<NT, CPT>(r, sr, k, rstd, sigma);
  }
  // token amax and the row-major copy of h (zero padding up to kp)
  float amax = 0.0f;
  uint16_t* hr = h_out + row * kp;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t j0 = ((int64_t)threadIdx.x + (int64_t)i * NT) * 8;
    if (j0 >= kp) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(r.v[i][e])), fabsf(hi_bf16(r.v[i][e]))));
    *reinterpret_cast<u32x4*>(hr + j0) = u32x4{r.v[i][0], r.v[i][1], r.v[i][2], r.v[i][3]};
  }
  amax = wave_max(amax);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) amax = fmaxf(amax, red[w]);
  // 2^p with amax * 2^p in [2^14, 2^15): p = 14 - floor(log2 amax), read off the exponent field; kept within the
  // normal exponent range so 2^p and 2^-p are plain f32 powers of two
  int p = 0;
  if (amax > 0.0f) {
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127;  // floor(log2 amax) for normal amax
    p = 14 - (e < -126 ? -126 : e);
    p = p > 126 ? 126 : p;
  }
  const float up = __uint_as_float((uint32_t)(p + 127) << 23);
  if (threadIdx.x == 0) xunscale[row] = __uint_as_float((uint32_t)(127 - p) << 23);
  // MFMA B-fragments: chunk of 8 consecutive k of this token sits in token tile row/16 at ((kt*4 + s)*64 + lane),
  // lane = 16 * ((k % 32) / 8) + row % 16
  const int64_t tile = row / 16;
  const int col = (int)(row % 16);
  const int64_t KT = kp / kKTile;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t j0 = ((int64_t)threadIdx.x + (int64_t)i * NT) * 8;
    if (j0 >= kp) continue;
    uint32_t packed[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f16x2 v;
      v[0] = (_Float16)__fmul_rn(lo_bf16(r.v[i][e]), up);
      v[1] = (_Float16)__fmul_rn(hi_bf16(r.v[i][e]), up);
      packed[e] = __builtin_bit_cast(uint32_t, v);
    }
    const int64_t kt = j0 / kKTile;
    const int s = (int)((j0 % kKTile) / 32), lhi = (int)((j0 % 32) / 8);
    xs[((tile * KT + kt) * 4 + s) * kWave + lhi * 16 + col] = u32x4{packed[0], packed[1], packed[2], packed[3]};
  }
}

// ------------------------------------------------------------------------------------------------------------------
// P2: partial t over one k-chunk, t_c[p][tok][j] = sum over k in chunk c of A_p[j][k] * h[tok][k].
// Workgroup (token tile, projection p, rank group jg of 16, chunk c): 16 waves take the chunk's 32-wide slices, issue
// all their loads (at most 8 slices each), run bf16 16x16x32 MFMAs and meet in LDS. The 16 x 16 partial is stored
// where the LoRA-up B-fragment wants it: element (rank j, token tok) of chunk c at
// [p][tile][j / 32][c][lane = ((j % 32) / 8) * 16 + tok][j % 8]. Ranks past r come out 0 (their A rows read as 0).
constexpr int kLoraWaves = 16;
constexpr int kLoraSlicesPerWave = 8;

struct LoraDownArgs {
  const uint16_t* A[kMaxProj];
  int32_t r[kMaxProj];
  int32_t nproj, jgmax, ks;
  int64_t m, k, kp, kc_width;
  const uint16_t* h;  // [mp][kp]
  int64_t h_bytes;
  float* t_part;
};

__global__ void __launch_bounds__(kLoraWaves * kWave) k_lora_down(LoraDownArgs a) {
  __shared__ f32x4 red[kLoraWaves][kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int64_t tile = blockIdx.x, ntiles = gridDim.x;
  int job = blockIdx.y;
  const int kc = job % a.ks;
  job /= a.ks;
  const int jg = job % a.jgmax;
  const int p = job / a.jgmax;
  const int r = a.r[p];
  const int j = jg * 16 + lane % 16;
  const int64_t tok = tile * 16 + lane % 16;
  const int64_t k0 = kc * a.kc_width, k1 = k0 + a.kc_width < a.k ? k0 + a.kc_width : a.k;
  const rsrc_t asrc = make_rsrc(a.A[p], (int64_t)r * a.k * 2), hsrc = make_rsrc(a.h, a.h_bytes);
  u32x4 av[kLoraSlicesPerWave], bv[kLoraSlicesPerWave];
#pragma unroll
  for (int i = 0; i < kLoraSlicesPerWave; ++i) {
    const int64_t kk = k0 + (int64_t)(i * kLoraWaves + wave) * 32 + (lane / 16) * 8;
    const bool in = kk < k1;
    av[i] = bload16(asrc, (in && j < r) ? (uint32_t)(((int64_t)j * a.k + kk) * 2) : kOutOfRange);
    bv[i] = bload16(hsrc, (in && tok < a.m) ? (uint32_t)((tok * a.kp + kk) * 2) : kOutOfRange);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kLoraSlicesPerWave; ++i)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[i]), __builtin_bit_cast(bf16x8, bv[i]),
                                                  acc, 0, 0, 0);
  red[wave][lane] = acc;
  __syncthreads();
  if (threadIdx.x < 256) {
    // thread (rank row jr, token column tc); D lane (jr/4)*16 + tc, element jr%4
    const int jr = threadIdx.x / 16, tc = threadIdx.x % 16;
    const int src = (jr / 4) * 16 + tc, q = jr % 4;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kLoraWaves; ++w) v += red[w][src][q];
    const int jj = jg * 16 + jr;
    const int L = ((jj % 32) / 8) * 16 + tc;
    a.t_part[((((int64_t)p * ntiles + tile) * kRankChunks + jj / 32) * a.ks + kc) * kWave * 8 + L * 8 + jj % 8] = v;
  }
}

// ------------------------------------------------------------------------------------------------------------------
// L: main streaming kernel.
//   TMT  token tiles of 16 in this launch
//   R    row groups (16 rows each) per workgroup; with SILU they are (gate, up) pairs: slot 2i = gate, 2i+1 = up
//   W    waves; wave w takes the contiguous k-tile range [w*KT/W, (w+1)*KT/W) for all R row groups
// Per k-tile and row group a lane loads one 16-byte code chunk and one dword of scales; per token tile and slice one
// 16-byte B-fragment. Loads of tile i+1 are issued before tile i is computed.
template <int TMT, int R>
struct TileBuf {
  u32x4 c[R];
  uint32_t sc[R];
  u32x4 b[TMT][4];
};

// Operand streams of one workgroup. Buffer descriptors are wave-uniform (SGPRs); each lane adds one 32-bit offset.
// Dead row-group slots have num_records = 0 and absent tokens an out-of-range offset, so their loads return zeros.
template <int TMT, int R>
struct Streams {
  rsrc_t c[R], s[R], b;
  uint32_t c_off, s_off, b_off[TMT];
};

template <int TMT, int R>
__device__ __forceinline__ void load_tile(TileBuf<TMT, R>& t, const Streams<TMT, R>& st, int64_t kt) {
  const int kc = __builtin_amdgcn_readfirstlane((int)(kt * kTileCodeBytes));
  const int ks = __builtin_amdgcn_readfirstlane((int)(kt * kTileScaleBytes));
  const int kb = __builtin_amdgcn_readfirstlane((int)(kt * 4 * kWave * 16));
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
}

template <int TMT, int R>
__device__ __forceinline__ void compute_tile(const TileBuf<TMT, R>& t, f32x4 (&acc)[R][TMT]) {
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
        acc[rr][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(f16x8, t.b[tt][s]), acc[rr][tt],
                                                              0, 0, 0);
    }
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
      for (int c = 1; c < a.ks; ++c) {  // k > 4096: the remaining chunks, in chunk order
        const uint32_t oc = off + (uint32_t)c * kWave * 32;
        s0 += __builtin_bit_cast(f32x4, bload16(tsrc, ok ? oc : kOutOfRange));
        s1 += __builtin_bit_cast(f32x4, bload16(tsrc, ok ? oc + 16 : kOutOfRange));
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

  // epilogue operands fetched now, consumed after the weight stream: per output the token's 2^-p and the residual
  // (unconditional loads: outputs the epilogue skips read a valid stand-in address instead)
  float xu[kOut];
  uint16_t res[kOut];
#pragma unroll
  for (int i = 0; i < kOut; ++i) {
    const int o = threadIdx.x + i * W * kWave;
    const int row = o % 16, tok = (o / 16) % mt, slot = o / (16 * mt);
    xu[i] = gload(a.xunscale + a.tok0 + tok);
    const uint16_t* rp = reinterpret_cast<const uint16_t*>(a.xunscale);
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
#pragma unroll
  for (int tt = 0; tt < TMT; ++tt)
    st.b_off[tt] = (tt * 16 + lane % 16 < mt) ? (uint32_t)((tt * KT * 4 * kWave + lane) * 16) : kOutOfRange;

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
      val[q] = sg * (s * xu[i]) + lm * red[W][rr][tt][ln][ii];
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
  // 32-bit buffer offsets: the row-major copy of h and every LoRA-B matrix stay below 2 GiB
  if (ceil_div(m, 16) * 16 * ceil_div(k, kKTile) * kKTile * 2 >= ((int64_t)1 << 31)) return QN_ERR_UNSUPPORTED;
  for (int p = 0; p < nproj; ++p)
    if ((int64_t)projs[p].n * projs[p].r * 2 >= ((int64_t)1 << 31)) return QN_ERR_UNSUPPORTED;

  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  const int64_t kp = ceil_div(k, kKTile) * kKTile;
  const int64_t mp = ceil_div(m, 16) * 16;
  u32x4* xs = reinterpret_cast<u32x4*>(ws + wl.xs);
  float* xunscale = reinterpret_cast<float*>(ws + wl.xunscale);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + wl.h);
  float* t_part = reinterpret_cast<float*>(ws + wl.t_part);
  int max_r = 0;
  for (int p = 0; p < nproj; ++p) max_r = projs[p].r > max_r ? projs[p].r : max_r;
  const int jgmax = 2 * (int)ceil_div(max_r, 32);  // whole 32-rank chunks, so every fragment element gets written
  const int ks = (int)lora_chunks(k);

  // P1
  const int vec_in = ((uintptr_t)x % 16 == 0) && (ldx % 8 == 0);
  if (run_prologue) {
    const int nt = norm_threads(kp);
    const int64_t cpt = ceil_div(ceil_div(kp, 8), nt);
    const int has_aqn = aqn ? 1 : 0;
    const uint16_t* g = aqn ? aqn->gamma : nullptr;
    const float* nz = aqn ? aqn->noise : nullptr;
    const int64_t nld = aqn ? aqn->noise_ld : 0;
    const float sg = aqn ? aqn->sigma : 0.f, ep = aqn ? aqn->eps : 0.f;
    const int vec_g = g && (uintptr_t)g % 16 == 0;
    const int vec_z = nz && (uintptr_t)nz % 16 == 0 && nld % 4 == 0;
#define QN_P1(NT_, CPT_)                                                                                          \
  hipLaunchKernelGGL((k_norm_convert<NT_, CPT_>), dim3((unsigned)m), dim3(NT_), 0, s, x, ldx, k, kp, has_aqn, g, nz, \
                     nld, sg, ep, vec_in, vec_g, vec_z, h, xs, xunscale)
    if (nt == 256) {
      if (cpt <= 1) QN_P1(256, 1);
      else if (cpt <= 2) QN_P1(256, 2);
      else if (cpt <= 4) QN_P1(256, 4);
      else if (cpt <= 8) QN_P1(256, 8);
      else QN_P1(256, 16);
    } else {
      QN_P1(1024, 16);
    }
#undef QN_P1
  }

  // P2
  if (run_prologue && max_r > 0) {
    LoraDownArgs la{};
    for (int p = 0; p < nproj; ++p) {
      la.A[p] = projs[p].lora_a;
      la.r[p] = projs[p].r;
    }
    la.nproj = nproj;
    la.jgmax = jgmax;
    la.ks = ks;
    la.m = m;
    la.k = k;
    la.kp = kp;
    la.kc_width = lora_chunk_width(k);
    la.h = h;
    la.h_bytes = mp * kp * 2;
    la.t_part = t_part;
    hipLaunchKernelGGL(k_lora_down, dim3((unsigned)(mp / 16), (unsigned)(nproj * jgmax * ks)),
                       dim3(kLoraWaves * kWave), 0, s, la);
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
  la.xunscale = xunscale;
  la.t_part = reinterpret_cast<const u32x4*>(t_part);
  la.t_bytes = (int64_t)(wl.total - wl.t_part);
  la.ks = ks;
  const bool silu = epilogue == QN_EPI_SILU_MUL;
  const int64_t nrg = silu ? 2 * ceil_div(projs[0].n, 16) : rg_total;
  if (nrg == 0 || !run_main) return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
  const int64_t KT = kp / kKTile;
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

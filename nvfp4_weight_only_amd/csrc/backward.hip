// Backward of the rollout layer's linear through the frozen NVFP4 weight.
//
// "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops" (technical review): §2.1
// the backbone W_hat is frozen and the gradients update the adapter A, B; they may still have to pass through the
// frozen projection to reach an earlier adapter; §6, steps 8-10 (loss, then the update of the trainable parameters).
// For y = s_g W_hat h + lambda B (A h) and the upstream gradient g = dL/dy:
//   u = B^T g,  t = A h                                        (per token, rank r)
//   dh = s_g W_hat^T g + lambda A^T u                          (the gradient through the frozen projection)
//   dA = lambda u^T h,  dB = lambda g^T t
// Kernels, all on the caller's stream:
//   k_bt       B^T [r][n8] bf16 (rows padded to a multiple of 8 with zeros), so both operands of u = B^T g run along
//              the contraction.
//   k_skinny   t and u: out[m][j] = sum_c X[m][c] Y[j][c] with bf16 16x16x32 MFMAs, 64 tokens per workgroup, the
//              contraction split over 8 waves and summed in a fixed tree.
//   k_dh       dh: workgroup tile 128 tokens x 512 input channels, stepping over the output rows 32 at a time. The
//              tiled NVFP4 weight holds 8 consecutive input channels per lane; the MFMA needs 8 consecutive output
//              rows, so each step dequantizes 2 row groups x 4 k-tiles (s_b * q, exact in bf16) and writes them to LDS
//              transposed, beside the 128 x 32 slice of g. Double-buffered, one barrier per step. The LoRA term and
//              s_g are applied in the epilogue.
//   k_outer    dA and dB: out[p][j] = sum over a chunk of tokens of X[m][p] T[m][j] (X = h or g in bf16, T = u or t
//              in f32 split into bf16 hi + lo parts); 64 rows of p per workgroup, tokens in chunks whose partial sums
//              k_outer_sum adds in chunk order (results do not depend on scheduling).
#include <cmath>

#include "qn_device.hpp"

namespace qn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                 0);
}

// Eight consecutive bf16 of a row at element c of [0, len): one 16-byte load when all eight are in range and the
// rows are 16-byte aligned (vec: base and row pitch), else element by element with zeros past len.
__device__ __forceinline__ u32x4 load8_bf16(const uint16_t* row, int64_t c, int64_t len, bool vec = true) {
  if (vec && c + 8 <= len) return gload(reinterpret_cast<const u32x4*>(row + c));
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = c + 2 * e < len ? gload(row + c + 2 * e) : 0u;
    const uint32_t hi = c + 2 * e + 1 < len ? gload(row + c + 2 * e + 1) : 0u;
    w[e] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// f32 values as bf16 hi + lo parts (t - hi is exact in f32: 16 significant bits kept)
__device__ __forceinline__ void split_bf16(const float (&v)[8], u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h0 = f32_to_bf16(v[2 * e]), h1 = f32_to_bf16(v[2 * e + 1]);
    const uint32_t l0 = f32_to_bf16(v[2 * e] - bf16_to_f32((uint16_t)h0));
    const uint32_t l1 = f32_to_bf16(v[2 * e + 1] - bf16_to_f32((uint16_t)h1));
    h[e] = h0 | (h1 << 16);
    l[e] = l0 | (l1 << 16);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// ---- B^T ------------------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_bt(const uint16_t* __restrict__ B, int64_t n, int r, int64_t n8,
                                            uint16_t* __restrict__ bt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over [r][n8]
  if (i >= (int64_t)r * n8) return;
  const int j = (int)(i / n8);
  const int64_t o = i % n8;
  bt[i] = o < n ? B[o * r + j] : (uint16_t)0;
}

// ---- t = A h, u = B^T g -----------------------------------------------------------------------------------------------
constexpr int kSkWaves = 8;
constexpr int kSkTT = 4;  // token tiles per workgroup

struct SkinnyArgs {
  const uint16_t* X;  // [M][ldx] bf16 (16-byte aligned rows)
  int64_t ldx;
  const uint16_t* Y;  // [R][ldy] bf16 (16-byte aligned rows)
  int64_t ldy;
  int64_t M, C;
  int32_t R;
  float* out;  // [M][R] f32
  int32_t vec_x;  // X rows 16-byte aligned
};

__global__ void __launch_bounds__(kSkWaves * kWave) k_skinny(SkinnyArgs a) {
  __shared__ f32x4 s_red[kSkWaves / 2][4][kSkTT][kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int64_t m0 = (int64_t)blockIdx.x * kSkTT * 16;
  const int njt = (a.R + 15) / 16;
  const int64_t nsl = ceil_div(a.C, 32);
  const int64_t sb = wave * nsl / kSkWaves, se = (wave + 1) * nsl / kSkWaves;
  f32x4 acc[4][kSkTT];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int tt = 0; tt < kSkTT; ++tt) acc[jt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lc = 8 * (lane / 16);
  for (int64_t sl = sb; sl < se; ++sl) {
    const int64_t c = sl * 32 + lc;
    u32x4 yv[4], xv[kSkTT];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = jt * 16 + lane % 16;
      yv[jt] = (jt < njt && j < a.R) ? load8_bf16(a.Y + (int64_t)j * a.ldy, c, a.C) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int tt = 0; tt < kSkTT; ++tt) {
      const int64_t m = m0 + tt * 16 + lane % 16;
      xv[tt] = m < a.M ? load8_bf16(a.X + m * a.ldx, c, a.C, a.vec_x) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt >= njt) break;
#pragma unroll
      for (int tt = 0; tt < kSkTT; ++tt) acc[jt][tt] = mfma_bf16(yv[jt], xv[tt], acc[jt][tt]);
    }
  }
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int tt = 0; tt < kSkTT; ++tt) mfma_settle(acc[jt][tt]);
  // waves' partial sums added in a fixed tree: (w, w + 4), then (w, w + 2), then (0, 1)
  for (int half = kSkWaves / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int tt = 0; tt < kSkTT; ++tt) s_red[wave - half][jt][tt][lane] = acc[jt][tt];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int tt = 0; tt < kSkTT; ++tt) acc[jt][tt] += s_red[wave][jt][tt][lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  // D lane l, element e: row (j) 4 (l/16) + e of the j-tile, column (token) l % 16 of the token tile
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int tt = 0; tt < kSkTT; ++tt) {
      const int64_t m = m0 + tt * 16 + lane % 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = jt * 16 + 4 * (lane / 16) + e;
        if (m < a.M && j < a.R) a.out[m * a.R + j] = acc[jt][tt][e];
      }
    }
}

// ---- dh = s_g W_hat^T g + lambda A^T u --------------------------------------------------------------------------------
constexpr int kDhWaves = 8;
constexpr int kDhTok = 128;   // tokens per workgroup (8 token tiles)
constexpr int kDhK = 512;     // input channels per workgroup (4 k-tiles); wave w takes 64 of them
constexpr int kDhPitch = 40;  // LDS row pitch (bf16): 32 rows of the step + 8 against bank conflicts

struct DhArgs {
  const uint16_t* g;  // [M][ldg] bf16
  int64_t ldg;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* s_g;
  const uint16_t* A;  // [r][K] bf16
  const float* u;     // [M][r] f32
  int64_t M, N, K, KT;
  int32_t r, ntb, nkb;
  float lambda;
  void* dh;
  int64_t lddh;
  int32_t dh_dtype;
  int32_t vec_g;  // g rows 16-byte aligned
};

// E2M1 codes (8 per dword) times the E4M3 block scale, exactly (s_b * q has at most 6 significant bits), as bf16
__device__ __forceinline__ void dequant8_bf16(uint32_t cw, uint32_t scale_byte, uint16_t (&o)[8]) {
  const f16x2 sh = __builtin_bit_cast(f16x2, scale_byte * 0x00800080u);  // E4M3 byte << 7 = E4M3 * 2^-8 in f16
  const f16x2 q[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 0) * sh,
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 1) * sh,
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 2) * sh,
                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 256.0f, 3) * sh};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    o[2 * p] = (uint16_t)(__float_as_uint((float)q[p][0]) >> 16);  // f16 -> f32 -> bf16: exact for these values
    o[2 * p + 1] = (uint16_t)(__float_as_uint((float)q[p][1]) >> 16);
  }
}

__global__ void __launch_bounds__(kDhWaves * kWave) k_dh(DhArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2][kDhK][kDhPitch];    // W_hat^T of the step: [k][n]
  __shared__ __attribute__((aligned(16))) uint16_t s_g[2][kDhTok][kDhPitch];  // g of the step: [token][n]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int tid = threadIdx.x;
  // workgroup -> (token block, k block): each XCD walks a contiguous range, k blocks fastest, so the workgroups an
  // XCD runs together share the token block's rows of g in its L2
  int tb, kb;
  {
    const int nwg = a.ntb * a.nkb, id = blockIdx.x;
    const int x = id % 8, q = nwg / 8, rem = nwg % 8;
    const int gi = x * q + (x < rem ? x : rem) + id / 8;
    tb = gi / a.nkb;
    kb = gi % a.nkb;
  }
  const int64_t t0 = (int64_t)tb * kDhTok, kbase = (int64_t)kb * kDhK;
  const int64_t NG = ceil_div(a.N, 16), NS = ceil_div(a.N, 32);
  const rsrc_t csrc = make_rsrc(a.codes, NG * a.KT * kTileCodeBytes);
  const rsrc_t ssrc = make_rsrc(a.scales, NG * a.KT * kTileScaleBytes);

  // the step's loads into registers: two (lane pair, slice) items of weights and one 16-byte piece of g per thread
  struct Regs {
    uint32_t c0[2], c1[2], sc[2];
    u32x4 gv;
  };
  auto item_of = [&](int q, int& rgl, int& ktl, int& lp, int& sd) {
    const int it = tid + q * kDhWaves * kWave;  // 0 .. 1023: [rg 2][k-tile 4][lane pair 32][slice 4]
    rgl = it >> 9;
    ktl = (it >> 7) & 3;
    lp = (it >> 2) & 31;
    sd = it & 3;
  };
  auto load_step = [&](Regs& R, int64_t st) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int rgl, ktl, lp, sd;
      item_of(q, rgl, ktl, lp, sd);
      const int64_t gg = 2 * st + rgl, kt = kb * 4 + ktl;
      const bool ok = gg < NG && kt < a.KT;
      const int L = 2 * lp;  // lanes L, L + 1 of the tile: rows L % 16 and L % 16 + 1, the same eight channels
      const uint32_t tile = ok ? (uint32_t)((gg * a.KT + kt)) : 0u;
      R.c0[q] = __builtin_amdgcn_raw_buffer_load_b32(csrc, ok ? tile * kTileCodeBytes + L * 16 + sd * 4 : kOutOfRange, 0, 0);
      R.c1[q] = __builtin_amdgcn_raw_buffer_load_b32(csrc, ok ? tile * kTileCodeBytes + (L + 1) * 16 + sd * 4 : kOutOfRange,
                                                     0, 0);
      // scale bytes of rows L % 16 and L % 16 + 1 for this slice and half: byte [row][h][s] = row * 8 + h * 4 + s
      const uint32_t so = tile * kTileScaleBytes + (L % 16) * 8 + ((L / 16) / 2) * 4 + sd;
      const uint32_t b0 = __builtin_amdgcn_raw_buffer_load_b8(ssrc, ok ? so : kOutOfRange, 0, 0);
      const uint32_t b1 = __builtin_amdgcn_raw_buffer_load_b8(ssrc, ok ? so + 8 : kOutOfRange, 0, 0);
      R.sc[q] = b0 | (b1 << 8);
    }
    const int row = tid >> 2, ch = tid & 3;
    const int64_t m = t0 + row, n = st * 32 + ch * 8;
    R.gv = (m < a.M && n < a.N) ? load8_bf16(a.g + m * a.ldg, n, a.N, a.vec_g) : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_step = [&](const Regs& R, int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int rgl, ktl, lp, sd;
      item_of(q, rgl, ktl, lp, sd);
      const int L = 2 * lp;
      uint16_t w0[8], w1[8];
      dequant8_bf16(R.c0[q], R.sc[q] & 0xFFu, w0);
      dequant8_bf16(R.c1[q], (R.sc[q] >> 8) & 0xFFu, w1);
      const int nl = rgl * 16 + (L % 16);             // even: rows nl, nl + 1 share one dword of the LDS row
      const int kl = ktl * 128 + 32 * sd + 8 * (L / 16);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t*>(&s_w[buf][kl + i][nl]) = (uint32_t)w0[i] | ((uint32_t)w1[i] << 16);
    }
    const int row = tid >> 2, ch = tid & 3;
    *reinterpret_cast<u32x4*>(&s_g[buf][row][ch * 8]) = R.gv;
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) acc[kk][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  Regs R;
  load_step(R, 0);
  store_step(R, 0);
  __syncthreads();
  for (int64_t st = 0; st < NS; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < NS) load_step(R, st + 1);
    // A: W_hat^T rows (channels) of this wave's 4 subtiles, 8 output rows n per lane; B: g, 8 n per lane per token
    u32x4 av[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      av[kk] = *reinterpret_cast<const u32x4*>(&s_w[buf][wave * 64 + kk * 16 + lane % 16][8 * (lane / 16)]);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(&s_g[buf][tt * 16 + lane % 16][8 * (lane / 16)]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc[kk][tt] = mfma_bf16(av[kk], bv, acc[kk][tt]);
    }
    if (st + 1 < NS) store_step(R, (int)((st + 1) & 1));
    __syncthreads();
  }

  // epilogue, one token tile at a time: lambda A^T u (D rows = channels 4 (l/16) + e, columns = tokens l % 16), then
  // s_g, store. The rows of A^T for this wave's channels are gathered once (at most two 32-rank chunks).
  const float sg = gload(a.s_g);
  const bool lora = a.r > 0 && a.lambda != 0.0f;
  u32x4 atv[2][4];
#pragma unroll
  for (int jc = 0; jc < 2; ++jc)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int j0 = jc * 32 + 8 * (lane / 16);
      const int64_t k = kbase + wave * 64 + kk * 16 + lane % 16;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok0 = lora && k < a.K && j0 + 2 * e < a.r, ok1 = lora && k < a.K && j0 + 2 * e + 1 < a.r;
        const uint32_t lo = ok0 ? gload(a.A + (int64_t)(j0 + 2 * e) * a.K + k) : 0u;
        const uint32_t hi = ok1 ? gload(a.A + (int64_t)(j0 + 2 * e + 1) * a.K + k) : 0u;
        w[e] = lo | (hi << 16);
      }
      atv[jc][kk] = u32x4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) mfma_settle(acc[kk][tt]);
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const int64_t m = t0 + tt * 16 + lane % 16;
    f32x4 la[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (lora) {
#pragma unroll
      for (int jc = 0; jc < 2; ++jc) {
        if (jc * 32 >= a.r) break;
        const int j0 = jc * 32 + 8 * (lane / 16);
        float uv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) uv[e] = (m < a.M && j0 + e < a.r) ? gload(a.u + m * a.r + j0 + e) : 0.0f;
        u32x4 hi, lo;
        split_bf16(uv, hi, lo);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          la[kk] = mfma_bf16(atv[jc][kk], hi, la[kk]);
          la[kk] = mfma_bf16(atv[jc][kk], lo, la[kk]);
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) mfma_settle(la[kk]);
    if (m >= a.M) continue;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int64_t k = kbase + wave * 64 + kk * 16 + 4 * (lane / 16);
      if (k >= a.K) continue;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = sg * acc[kk][tt][e] + a.lambda * la[kk][e];
      if (a.dh_dtype == QN_F32) {
        float* p = reinterpret_cast<float*>(a.dh) + m * a.lddh + k;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k + e < a.K) p[e] = o[e];
      } else {
        uint16_t* p = reinterpret_cast<uint16_t*>(a.dh) + m * a.lddh + k;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k + e < a.K) p[e] = f32_to_bf16(o[e]);
      }
    }
  }
}

// ---- dA, dB: partial sums of X^T T over token chunks --------------------------------------------------------------
constexpr int kOuWaves = 4;
constexpr int kOuP = 64;        // rows of p per workgroup (wave w: 16)
constexpr int kOuPitchX = 40;   // LDS pitch of the transposed X slice (bf16): 32 tokens + 8
constexpr int kOuPitchT = 36;   // LDS pitch of the transposed T slice (f32): 32 tokens + 4

struct OuterArgs {
  const uint16_t* X;  // [M][ldx] bf16
  int64_t ldx;
  const float* T;     // [M][r] f32
  int64_t M, P;
  int32_t r, nchunk;
  int64_t chunk;      // tokens per chunk (a multiple of 32)
  float* part;        // [nchunk][P][r] f32
  int32_t vec_x;      // X rows 16-byte aligned
};

__global__ void __launch_bounds__(kOuWaves * kWave) k_outer(OuterArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kOuP][kOuPitchX];   // X^T slice: [p][token]
  __shared__ __attribute__((aligned(16))) float s_t[64][kOuPitchT];        // T^T slice: [j][token]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int tid = threadIdx.x;
  const int64_t p0 = (int64_t)blockIdx.x * kOuP;
  const int ch = blockIdx.y;
  const int64_t mb = (int64_t)ch * a.chunk, me = mb + a.chunk < a.M ? mb + a.chunk : a.M;
  const int njt = (a.r + 15) / 16;
  f32x4 acc[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t m0 = mb; m0 < me; m0 += 32) {
    // X slice: thread -> token tid / 8, eight channels 8 (tid % 8); T slice: token tid / 8, ranks 8 (tid % 8)
    {
      const int row = tid >> 3, c8 = tid & 7;
      const int64_t m = m0 + row, p = p0 + c8 * 8;
      const u32x4 xv = (m < me && p < a.P) ? load8_bf16(a.X + m * a.ldx, p, a.P, a.vec_x) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_x[c8 * 8 + 2 * e][row] = (uint16_t)(xv[e] & 0xFFFFu);
        s_x[c8 * 8 + 2 * e + 1][row] = (uint16_t)(xv[e] >> 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = c8 * 8 + e;
        s_t[j][row] = (m < me && j < a.r) ? gload(a.T + m * a.r + j) : 0.0f;
      }
    }
    __syncthreads();
    const u32x4 xa = *reinterpret_cast<const u32x4*>(&s_x[wave * 16 + lane % 16][8 * (lane / 16)]);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt >= njt) break;
      float tv[8];
      const float* tp = &s_t[jt * 16 + lane % 16][8 * (lane / 16)];
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[e] = tp[e];
      u32x4 hi, lo;
      split_bf16(tv, hi, lo);
      acc[jt] = mfma_bf16(xa, hi, acc[jt]);
      acc[jt] = mfma_bf16(xa, lo, acc[jt]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) mfma_settle(acc[jt]);
  // D lane l, element e: row p = wave * 16 + 4 (l/16) + e, column j = jt * 16 + l % 16
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    if (jt >= njt) break;
    const int j = jt * 16 + lane % 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t p = p0 + wave * 16 + 4 * (lane / 16) + e;
      if (p < a.P && j < a.r) a.part[((int64_t)ch * a.P + p) * a.r + j] = acc[jt][e];
    }
  }
}

// out = lambda * (sum of the chunk partials in chunk order), [P][r] or transposed [r][P]
__global__ void __launch_bounds__(256) k_outer_sum(const float* __restrict__ part, int nchunk, int64_t P, int r,
                                                   float lambda, float* __restrict__ out, int transposed) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= P * r) return;
  float s = part[i];
  for (int c = 1; c < nchunk; ++c) s += part[(int64_t)c * P * r + i];
  const int64_t p = i / r;
  const int j = (int)(i % r);
  out[transposed ? (int64_t)j * P + p : i] = lambda * s;
}

// ---- host side ---------------------------------------------------------------------------------------------------
struct BwdWs {
  size_t bt, t, u, part, total;
};

inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

int outer_chunks(int64_t m, int64_t P) {
  // about 512 workgroups, each chunk a multiple of 32 tokens
  const int64_t pb = ceil_div(P, kOuP);
  int64_t nc = ceil_div(512, pb);
  const int64_t maxc = ceil_div(m, 32);
  if (nc > maxc) nc = maxc;
  if (nc < 1) nc = 1;
  return (int)nc;
}

BwdWs bwd_layout(int64_t m, int64_t n, int64_t k, int r) {
  BwdWs w;
  size_t off = 0;
  const int64_t n8 = ceil_div(n, 8) * 8;
  w.bt = off;   off = al256(off + (size_t)r * n8 * 2);
  w.t = off;    off = al256(off + (size_t)m * r * 4);
  w.u = off;    off = al256(off + (size_t)m * r * 4);
  const size_t pb = (size_t)outer_chunks(m, n) * n * r * 4, pa = (size_t)outer_chunks(m, k) * k * r * 4;
  w.part = off; off = al256(off + (pb > pa ? pb : pa));
  w.total = off;
  return w;
}

inline bool al(const void* p, size_t b) { return (uintptr_t)p % b == 0; }

}  // namespace
}  // namespace qn

using namespace qn;

extern "C" size_t nvfp4_lora_linear_backward_workspace(int64_t m, int64_t n, int64_t k, int32_t r) {
  if (m <= 0 || n <= 0 || k <= 0 || r < 0) return 0;
  return bwd_layout(m, n, k, r).total;
}

extern "C" qn_status nvfp4_lora_linear_backward(const uint16_t* g, int64_t m, int64_t n, int64_t ldg, const uint16_t* h,
                                                int64_t k, int64_t ldh, const uint8_t* codes,
                                                const uint8_t* block_scales, const float* tensor_scale,
                                                const uint16_t* lora_a, const uint16_t* lora_b, int32_t r,
                                                float lambda, void* dh, int32_t dh_dtype, int64_t lddh, float* d_a,
                                                float* d_b, void* workspace, size_t workspace_bytes, void* stream) {
  if (m < 0 || n < 0 || k < 0 || k % 16 != 0 || r < 0) return QN_ERR_SHAPE;
  if (r > 64) return QN_ERR_UNSUPPORTED;
  if (!std::isfinite(lambda)) return QN_ERR_VALUE;
  if (dh && dh_dtype != QN_BF16 && dh_dtype != QN_F32) return QN_ERR_VALUE;
  if (m == 0 || n == 0 || k == 0) return QN_OK;
  if (!g) return QN_ERR_NULL;
  if (ldg < n || (dh && lddh < k)) return QN_ERR_SHAPE;
  if (!al(g, 2)) return QN_ERR_ALIGN;
  const bool need_h = r > 0 && (d_a || d_b);
  if (need_h && !h) return QN_ERR_NULL;
  if (need_h && (ldh < k)) return QN_ERR_SHAPE;
  if (need_h && !al(h, 2)) return QN_ERR_ALIGN;
  if (r > 0 && (!lora_a || !lora_b)) return QN_ERR_NULL;
  if (r > 0 && (!al(lora_a, 16) || !al(lora_b, 2))) return QN_ERR_ALIGN;
  if (dh && (!codes || !block_scales || !tensor_scale)) return QN_ERR_NULL;
  if (dh && (!al(codes, 16) || !al(block_scales, 4) || !al(tensor_scale, 4))) return QN_ERR_ALIGN;
  const BwdWs wl = bwd_layout(m, n, k, r);
  if (r > 0 && (!workspace || workspace_bytes < wl.total)) return QN_ERR_WORKSPACE;
  if (r > 0 && !al(workspace, 256)) return QN_ERR_ALIGN;
  const int64_t NG = ceil_div(n, 16), KT = ceil_div(k, kKTile);
  if (NG * KT * kTileCodeBytes >= ((int64_t)1 << 31)) return QN_ERR_UNSUPPORTED;  // 32-bit buffer offsets
  if (ceil_div(m, kDhTok) * ceil_div(k, kDhK) >= ((int64_t)1 << 31)) return QN_ERR_UNSUPPORTED;

  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  uint16_t* bt = r > 0 ? reinterpret_cast<uint16_t*>(ws + wl.bt) : nullptr;
  float* tv = r > 0 ? reinterpret_cast<float*>(ws + wl.t) : nullptr;
  float* uv = r > 0 ? reinterpret_cast<float*>(ws + wl.u) : nullptr;
  float* part = r > 0 ? reinterpret_cast<float*>(ws + wl.part) : nullptr;
  const int64_t n8 = ceil_div(n, 8) * 8;
  const int32_t vec_g = al(g, 16) && ldg % 8 == 0, vec_h = h && al(h, 16) && ldh % 8 == 0;
  if (r > 0) {
    // u = B^T g (for dh's LoRA term and dA), t = A h (for dB)
    if (dh || d_a) {
      hipLaunchKernelGGL(k_bt, dim3((unsigned)ceil_div((int64_t)r * n8, 256)), dim3(256), 0, s, lora_b, n, (int)r, n8, bt);
      SkinnyArgs sa{g, ldg, bt, n8, m, n, r, uv, vec_g};
      hipLaunchKernelGGL(k_skinny, dim3((unsigned)ceil_div(m, kSkTT * 16)), dim3(kSkWaves * kWave), 0, s, sa);
    }
    if (d_b) {
      SkinnyArgs sa{h, ldh, lora_a, k, m, k, r, tv, vec_h};
      hipLaunchKernelGGL(k_skinny, dim3((unsigned)ceil_div(m, kSkTT * 16)), dim3(kSkWaves * kWave), 0, s, sa);
    }
  }
  if (dh) {
    DhArgs da{};
    da.g = g;
    da.ldg = ldg;
    da.codes = codes;
    da.scales = block_scales;
    da.s_g = tensor_scale;
    da.A = r > 0 ? lora_a : nullptr;
    da.u = uv;
    da.M = m;
    da.N = n;
    da.K = k;
    da.KT = KT;
    da.r = r;
    da.ntb = (int32_t)ceil_div(m, kDhTok);
    da.nkb = (int32_t)ceil_div(k, kDhK);
    da.lambda = lambda;
    da.dh = dh;
    da.lddh = lddh;
    da.dh_dtype = dh_dtype;
    da.vec_g = vec_g;
    hipLaunchKernelGGL(k_dh, dim3((unsigned)(da.ntb * da.nkb)), dim3(kDhWaves * kWave), 0, s, da);
  }
  if (r > 0 && d_b) {  // dB [n][r] = lambda g^T t
    const int nc = outer_chunks(m, n);
    OuterArgs oa{g, ldg, tv, m, n, r, nc, ceil_div(ceil_div(m, nc), 32) * 32, part, vec_g};
    hipLaunchKernelGGL(k_outer, dim3((unsigned)ceil_div(n, kOuP), (unsigned)nc), dim3(kOuWaves * kWave), 0, s, oa);
    hipLaunchKernelGGL(k_outer_sum, dim3((unsigned)ceil_div(n * r, 256)), dim3(256), 0, s, part, nc, n, (int)r, lambda,
                       d_b, 0);
  }
  if (r > 0 && d_a) {  // dA [r][k] = lambda u^T h (computed as [k][r], stored transposed)
    const int nc = outer_chunks(m, k);
    OuterArgs oa{h, ldh, uv, m, k, r, nc, ceil_div(ceil_div(m, nc), 32) * 32, part, vec_h};
    hipLaunchKernelGGL(k_outer, dim3((unsigned)ceil_div(k, kOuP), (unsigned)nc), dim3(kOuWaves * kWave), 0, s, oa);
    hipLaunchKernelGGL(k_outer_sum, dim3((unsigned)ceil_div(k * r, 256)), dim3(256), 0, s, part, nc, k, (int)r, lambda,
                       d_a, 1);
  }
  return hipGetLastError() == hipSuccess ? QN_OK : QN_ERR_HIP;
}

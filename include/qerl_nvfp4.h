/* qerl_nvfp4.h — C ABI of the MI355X (gfx950) NVFP4 + LoRA + AQN-RMSNorm rollout-decode library.
 *
 * The operations follow the QeRL papers' decode linear layer as described in
 *   "QeRL: When Quantized Weights Help Reinforcement Learning, and Where the Evidence Stops" (technical review,
 *   zhongzhuzhou.org; cited below as [review §n]) and its Chinese counterpart "QeRL 阅读笔记".
 *
 * Conventions for every entry point:
 *   - Buffer pointers are DEVICE pointers (hipMalloc / torch CUDA tensors) unless a comment says "host".
 *     bf16 tensors are passed as uint16_t bit patterns, E2M1 codes and E4M3 scales as uint8_t.
 *   - The caller owns every buffer. The library allocates no device memory; scratch space comes from `workspace`
 *     (nvfp4_lora_linear_noalloc uses one device array of the library instead, see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls only enqueue work on it and
 *     return; results are ready when the stream reaches that point.
 *   - Errors: arguments are validated on the host before anything is launched; a failed validation returns a
 *     status other than QN_OK and enqueues nothing. QN_ERR_HIP reports a failed launch. Nothing is printed and
 *     nothing aborts. Conditions seen on the device are reported through an optional device flag word.
 *   - Thread safety: calls on different streams may run concurrently; the library keeps no mutable global state
 *     (except nvfp4_lora_linear_noalloc's shared scratch array, see there).
 *   - Empty inputs (m == 0 or n == 0) are valid and enqueue nothing.
 */
#ifndef QERL_NVFP4_H
#define QERL_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QN_OK = 0,
  QN_ERR_NULL = 1,        /* a required pointer is NULL */
  QN_ERR_SHAPE = 2,       /* negative size, k % 16 != 0, leading dimension too small, mismatched projections */
  QN_ERR_ALIGN = 3,       /* a pointer is not aligned as documented */
  QN_ERR_VALUE = 4,       /* a scalar is out of range (negative or non-finite sigma/eps/lambda, bad enum) */
  QN_ERR_WORKSPACE = 5,   /* workspace is NULL or smaller than nvfp4_lora_linear_workspace() */
  QN_ERR_UNSUPPORTED = 6, /* a valid request this library does not implement (e.g. LoRA rank > 64, > 4 projections) */
  QN_ERR_HIP = 7          /* a HIP launch failed */
} qn_status;

/* Layouts of a packed NVFP4 weight W [n x k] (row n = output channel, k = input channel).
 *
 * QN_LAYOUT_ROWMAJOR (the canonical layout; what the pages call packing into "the layout the kernel needs" is the
 * tiled one below, this one is for exchange and checking):
 *   codes  [n][k/2] bytes: byte j of row n holds element 2j in bits 3:0 and element 2j+1 in bits 7:4;
 *   scales [n][k/16] bytes: E4M3 block scale of elements 16b .. 16b+15 of row n (blocks run along k) [review §3.1].
 *   Total n*k/2 + n*k/16 = 9P/16 bytes [review §3.1, M_NVFP4 equation], plus the f32 tensor scale.
 *
 * QN_LAYOUT_TILED (what nvfp4_lora_linear reads): rows are padded to np = ceil(n/16)*16 and k to
 * kp = ceil(k/128)*128 with zero codes and zero scales. For row group g = n/16 and k-tile t = k/128:
 *   codes  tile (g, t) is 1024 bytes at ((g * kp/128 + t) * 1024); its 16-byte lane chunk L (L = 0..63) holds four
 *          little-endian dwords, dword s (s = 0..3) = the 8 codes of row 16g + L%16, elements
 *          128t + 32s + 8(L/16) .. +7, nibble order as in the row-major layout;
 *   scales tile (g, t) is 128 bytes at ((g * kp/128 + t) * 128): byte [r][h][s] (r = 0..15, h = 0..1, s = 0..3) is the
 *          scale of row 16g + r, elements 128t + 32s + 16h .. +15.
 *   Sizes: nvfp4_tiled_codes_bytes(n, k) and nvfp4_tiled_scales_bytes(n, k). Codes must be 16-byte aligned,
 *   scales 4-byte aligned. The permutation is chosen so that one 16-byte load per lane feeds four 16x16x32 MFMA
 *   A-fragments and every wave-wide load is one contiguous 1 KiB.
 */
typedef enum { QN_LAYOUT_ROWMAJOR = 0, QN_LAYOUT_TILED = 1 } qn_layout;

/* Output element type of a projection. */
typedef enum { QN_BF16 = 0, QN_F32 = 1 } qn_dtype;

/* Epilogues of nvfp4_lora_linear. */
typedef enum {
  QN_EPI_NONE = 0,
  /* SwiGLU gating before Down [review §5.1]: requires nproj == 2 with equal n; writes silu(y_0) * y_1 into projs[0].y
   * (projs[1].y is ignored and may be NULL). silu(v) = v / (1 + exp(-v)). */
  QN_EPI_SILU_MUL = 1
} qn_epilogue;

/* Phase flags, OR-ed into the `epilogue` argument of nvfp4_lora_linear. A call runs a prologue (the norm/convert and
 * the LoRA-down kernels, which fill the workspace) and then the main kernel (the weight stream and its epilogue).
 * A caller may split one call into two to place events or other work between the phases: first PROLOGUE_ONLY, then
 * MAIN_ONLY with the same arguments and workspace (the workspace must not be touched in between). */
#define QN_RUN_PROLOGUE_ONLY 0x100
#define QN_RUN_MAIN_ONLY 0x200

/* AQN-RMSNorm parameters [review §5.1 and §5.2]: h = u * (gamma + sigma * noise), u = x / sqrt(mean(x^2) + eps).
 * The clean scale gamma is only read, never written, so every call draws afresh around it (noise replacement,
 * [review §9.1]). */
typedef struct {
  const uint16_t* gamma; /* [d] bf16 norm scale (device) */
  const float* noise;    /* NULL (no noise) or standard-normal noise: [d] shared by all rows if noise_ld == 0, else
                            row i uses noise + i * noise_ld (device, f32) */
  int64_t noise_ld;
  float sigma;           /* noise standard deviation for this stage, >= 0 (see aqn_sigma); 0 gives plain RMSNorm */
  float eps;             /* >= 0, added to the mean square */
  /* Noise drawn on the device instead of read (draw != 0; noise must then be NULL): the same values aqn_noise
   * writes for (seed, subseed, row_offset, draw_rows), generated where the norm consumes them. */
  int32_t draw;
  uint64_t seed, subseed;
  uint64_t row_offset;   /* draw index of row 0 */
  int64_t draw_rows;     /* >= 0: rows per draw (e.g. the tokens of one response); 0 = one draw for every row */
} qn_aqn;

/* One projection consuming the shared activation: y = s_g * W_hat(codes, scales) x + lambda * B (A x)
 * [review §2.1, forward map], with optional residual and output broadcast. */
typedef struct {
  const uint8_t* codes;        /* QN_LAYOUT_TILED codes of W [n x k] (16-byte aligned) */
  const uint8_t* block_scales; /* QN_LAYOUT_TILED E4M3 block scales (4-byte aligned) */
  const float* tensor_scale;   /* one f32 s_g (device) */
  int64_t n;                   /* output channels */
  const uint16_t* lora_a;      /* [r][k] bf16 row-major, or NULL for no LoRA branch */
  const uint16_t* lora_b;      /* [n][r] bf16 row-major, or NULL for no LoRA branch */
  int32_t r;                   /* LoRA rank, 0..64 (0 = no branch) */
  float lambda;                /* adapter multiplier, applied as is (not divided by r) */
  void* y;                     /* output [m][ldy] of type y_dtype */
  int32_t y_dtype;             /* qn_dtype */
  int64_t ldy;                 /* output row stride in elements */
  const uint16_t* residual;    /* NULL or bf16 [m][ld_res] added to y before rounding; may alias y */
  int64_t ld_res;
  /* Output broadcast (grouped-query attention with the score computation excluded: each key/value head's vector is
   * copied to the `y_repeat` query heads of its group). 0 or 1 = off. When on, output element j of row i goes to
   * y[i*ldy + ((j / head_dim) * y_repeat + g) * head_dim + j % head_dim] for g = 0..y_repeat-1. */
  int32_t y_repeat;
  int32_t head_dim;
} qn_proj;

/* ---------------------------------------------------------------------------------------------------------------- */

/* Quantize a bf16 weight to NVFP4 [review §3.1: reconstruction w = s_g * s_b * q, q = argmin over the E2M1 grid of
 * |w - s_g s_b q| for fixed scales].
 *   w [n][ldw] bf16 (device), k % 16 == 0, ldw >= k.
 *   scale_mode 0: compute the scales by the amax rule (s_g = amax(|W|) / (6 * 448) in f32, or 1 if W == 0;
 *                 s_b = E4M3 round-to-nearest-even, saturating, of f32(amax_b / f32(6 * s_g))) and write them;
 *   scale_mode 1: read caller-fixed scales from block_scales (same layout as the output codes) and *tensor_scale;
 *                 they must be finite and non-negative.
 *   Codes: nearest E2M1 value under the fixed scales; exact midpoints go to the even code (mantissa bit 0); the sign
 *   is copied from w (a negative weight that rounds to zero gets code 8). Non-finite weights are left out of the
 *   amax, get code 0 and set bit 0 of *d_flags (if d_flags != NULL; the caller zeroes it beforehand).
 *   layout: qn_layout of codes and block_scales (the tiled layout also writes its zero padding).
 *   Launches four small kernels on `stream`; tensor_scale is used as scratch until the last one. */
qn_status nvfp4_quantize(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, int32_t scale_mode, int32_t layout,
                         uint8_t* codes, uint8_t* block_scales, float* tensor_scale, int32_t* d_flags, void* stream);

/* Bytes of the tiled codes / scales of an [n x k] weight (host, pure). */
size_t nvfp4_tiled_codes_bytes(int64_t n, int64_t k);
size_t nvfp4_tiled_scales_bytes(int64_t n, int64_t k);

/* Reconstruct W_hat = s_g * s_b * q [review §3.1] into f32 w_out [n][ldo]: the exact product rounded once to f32
 * (s_b * q is exact in f32). codes/block_scales in `layout`. */
qn_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* block_scales, const float* tensor_scale, int64_t n,
                           int64_t k, int32_t layout, float* w_out, int64_t ldo, void* stream);

/* MXFP4 quantizer, the OCP Microscaling FP4 format the papers calibrate and compare beside NVFP4 ["QeRL 阅读笔记" §3.1;
 * the pages give no more detail, so the OCP MX v1.0 definition is the reading]: blocks of 32 consecutive weights along
 * k share one E8M0 scale X = 2^(E - 127), E = floor(log2(block amax)) - 2 (2 = the largest E2M1 exponent) kept within
 * 0..254 (0 for a block without a nonzero finite weight); each element is the E2M1 code nearest to w / X (ties to the
 * even code, saturating at 6), with the sign of w. Non-finite weights are left out of the amax, get code 0 and set
 * bit 0 of *d_flags (if not NULL; the caller zeroes it beforehand).
 *   w [n][ldw] bf16 (device), k % 32 == 0, ldw >= k.
 *   layout QN_LAYOUT_ROWMAJOR: the canonical MX layout, codes [n][k/2] (packed as for NVFP4) and E8M0 scales
 *     [n][k/32] (mxfp4_scales_bytes); tensor_scale is not used (may be NULL).
 *   layout QN_LAYOUT_TILED: the same weight written exactly in the NVFP4 tiled form that nvfp4_lora_linear and the
 *     backward read (so every kernel serves MXFP4 weights): with E_ref = (largest E of the tensor) - 8, each 16-weight
 *     half of a block gets the E4M3 block scale 2^(E - E_ref) and *tensor_scale = 2^(E_ref - 127), so that
 *     s_g * s_b * q = X * q bit for bit. A block whose E is more than 17 below the largest cannot be written so: bit 1
 *     of *d_flags is set and that block's values are wrong (an error for the caller). codes and block_scales sized by
 *     nvfp4_tiled_codes_bytes / nvfp4_tiled_scales_bytes; tensor_scale is scratch until the last of four kernels.
 * Errors: QN_ERR_SHAPE (k % 32 != 0, ldw < k, negative sizes), QN_ERR_VALUE (layout), QN_ERR_NULL, QN_ERR_ALIGN (codes
 * 16-byte, tensor_scale and d_flags 4-byte aligned). */
qn_status mxfp4_quantize(const uint16_t* w, int64_t n, int64_t k, int64_t ldw, int32_t layout, uint8_t* codes,
                         uint8_t* scales, float* tensor_scale, int32_t* d_flags, void* stream);

/* Bytes of the canonical MXFP4 scales of an [n x k] weight (host, pure; 0 unless k % 32 == 0). */
size_t mxfp4_scales_bytes(int64_t n, int64_t k);

/* W_hat = X * q from the canonical MXFP4 layout into f32 w_out [n][ldo] (exact, rounded once to f32). */
qn_status mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k, float* w_out,
                           int64_t ldo, void* stream);

/* AQN-RMSNorm [review §5.1]: h = bf16(x * rstd * (gamma + sigma * noise)), rstd = 1 / sqrt(sum_j x_j^2 / d + eps),
 * per row, f32 arithmetic, round-to-nearest-even to bf16.  x [m][ldx] bf16, h [m][ldh] bf16 (device). */
qn_status aqn_rmsnorm(const uint16_t* x, int64_t m, int64_t d, int64_t ldx, const qn_aqn* aqn, uint16_t* h,
                      int64_t ldh, void* stream);

/* Standard-normal noise for AQN drawn from a seed [review §5.1 and §9.1: Gaussian noise on the norm scale at every
 * call; the pages leave the generator and the scope of a draw open]. Row i (0 <= i < m) takes draw index
 * r = row_offset + i / draw_rows (draw_rows > 0), or r = row_offset for every row (draw_rows == 0). Columns 8c .. 8c+7
 * of draw r come from one Philox4x64-10 block (Salmon, Moraes, Dror and Shaw, SC 2011) at counter (c, r, 0, 0)
 * under key (seed, subseed); its eight 32-bit words w0..w7 (w2q, w2q+1 = low, high half of output word q) give
 * columns 8c+2p, 8c+2p+1 by the Box-Muller transform: u(w) = ((w >> 9) + 1/2) 2^-23, rho = sqrt(-2 ln u(w2p)),
 * eps = rho cos(2 pi u(w2p+1)), rho sin(2 pi u(w2p+1)), in f32 (a few ulp from the exactly rounded values).
 * eps: [m][ld] f32 (device, 4-byte aligned), ld >= d. Errors: QN_ERR_SHAPE (m, d < 0, ld < d, draw_rows < 0),
 * QN_ERR_NULL, QN_ERR_ALIGN; nothing is launched on an error. */
qn_status aqn_noise(uint64_t seed, uint64_t subseed, uint64_t row_offset, int64_t draw_rows, int64_t m, int64_t d,
                    float* eps, int64_t ld, void* stream);

/* Workspace bytes nvfp4_lora_linear needs for these arguments (host, pure).
 * The workspace must be zero-filled before its first use (hipMemset once, or allocated zeroed). Every call leaves
 * its control words (split-k arrival counters, the prologue's LoRA-down arrival counters, the fused decode kernel's
 * counter and LoRA-down partials) zero again; they sit at the start of the workspace, at the same offsets for every
 * call, so a workspace can be reused by any later call ordered after it, whatever its shapes; calls that may run at
 * the same time need workspaces of their own. */
size_t nvfp4_lora_linear_workspace(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj);

/* The rollout-decode linear layer [review §2.1 forward map, §3.2, §5.1]:
 *   h = aqn ? AQN-RMSNorm(x) rounded to bf16 : x
 *   y_p = s_g,p * W_hat_p h + lambda_p * B_p (A_p h) (+ residual_p), for p = 0 .. nproj-1, then the epilogue.
 * One norm feeds all projections of the call (Q/K/V share the attention norm, Gate/Up the feed-forward norm,
 * [review §5.1]). x [m][ldx] bf16 with ldx >= k; k % 16 == 0; 1 <= nproj <= 4; all projections share k.
 * Activations enter the contraction as f16 after an exact per-token power-of-two rescale (see the library notes);
 * accumulation is f32. `projs` and `aqn` are host pointers to structs holding device pointers. */
qn_status nvfp4_lora_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                            const qn_proj* projs, int32_t nproj, int32_t epilogue, void* workspace,
                            size_t workspace_bytes, void* stream);

/* The same call on MXFP4 weights in the canonical MX layout (mxfp4_quantize with QN_LAYOUT_ROWMAJOR: codes [n][k/2],
 * E8M0 scales [n][k/32] in block_scales; tensor_scale unused, may be NULL), y = X q h + lambda B (A h) ["QeRL 阅读笔记"
 * §3.1 (MXFP4) with the forward map of review §2.1], run on CDNA4's scaled FP4 x FP8 matrix instruction, which takes
 * the E2M1 codes and their E8M0 scales as they are stored. The activations h (bf16, after the optional AQN-RMSNorm)
 * enter it as two E4M3 parts with one E8M0 exponent per 32 values along k: hi = E4M3(h / 2^s_hi) with the block's
 * largest |h| / 2^s_hi in [128, 256), lo = E4M3((h - hi 2^s_hi) / 2^s_lo) likewise from the remainders (round to
 * nearest even); hi 2^s_hi + lo 2^s_lo equals h for every value within a factor 2^10 of the largest magnitude in its
 * block, and differs from h by less than 2^-19 of that magnitude otherwise. Products and sums are f32; the LoRA branch,
 * the norm, epilogues, residual and broadcast are those of nvfp4_lora_linear. One kernel serves every token count
 * (tiles of 128 tokens, so it is meant for prefill; decode-sized calls are faster through the exact tiled form and
 * nvfp4_lora_linear). Errors as nvfp4_lora_linear, and QN_ERR_SHAPE for k % 32 != 0. Workspace: zero-filled before
 * its first use, mxfp4_lora_linear_workspace bytes, left with its control words zero (as for nvfp4_lora_linear). */
size_t mxfp4_lora_linear_workspace(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj);
qn_status mxfp4_lora_linear(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                            const qn_proj* projs, int32_t nproj, int32_t epilogue, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Kernel choice for nvfp4_lora_linear_opts. A call runs one of the streaming kernels below; the library picks one
 * from the token count and the shapes (QN_KERNEL_AUTO, what nvfp4_lora_linear does). Naming another one runs the same
 * computation, to the same accuracy bound, on that kernel: for checks of each kernel on the same inputs and for
 * timing them side by side. */
typedef enum {
  QN_KERNEL_AUTO = 0,    /* the library's choice */
  QN_KERNEL_GENERAL = 1, /* the general streaming kernel, one launch per 128 tokens; any m */
  QN_KERNEL_DECODE = 2,  /* the decode streaming kernel (activations held in LDS, optional split k); m <= 32 and a
                            split of the rows and k that fits its LDS, else QN_ERR_UNSUPPORTED */
  QN_KERNEL_MANY = 3,    /* the many-token MFMA kernel; m > 128, else QN_ERR_UNSUPPORTED */
  QN_KERNEL_FUSED = 4,   /* the decode kernel with the norm, the activation conversion and the LoRA-down folded in:
                            one launch per call; m <= 16, a cut that fits its LDS (with the norm: the whole row in one
                            k-chunk, k <= 3968), not with the phase flags, else QN_ERR_UNSUPPORTED. AUTO does not
                            take it: on the 7B decode shapes it measured slower than the prologue and the other
                            kernels at 1 to 16 tokens. */
  QN_KERNEL_WIDE = 5     /* the decode streaming kernel for 17 to 64 tokens (activations streamed through LDS in
                            passes, every activation tile shared by all row groups of a workgroup, optional split
                            k); m in 17..64, else QN_ERR_UNSUPPORTED. AUTO takes it at 17 to 64 tokens for calls
                            with at least 24 MB of packed weights (the wide feed-forward and long-row projections);
                            a split k needs at most 256 row blocks of 5 row units. At 65 to 128 tokens AUTO runs
                            such a call as sub-calls of at most 64 tokens on it, one after another on the stream
                            (not a call split into its phases); the workspace size covers them. */
} qn_kernel;

/* Explicit options of one nvfp4_lora_linear_opts call. Zero-initialised, it asks for the library's defaults. These
 * are the only inputs besides the arguments that change which kernel a call runs: the library reads no environment
 * variables and keeps no settings between calls. */
typedef struct {
  int32_t kernel;         /* qn_kernel */
  int32_t decode_kchunks; /* QN_KERNEL_DECODE / _FUSED / _WIDE: k-chunks of the split-k cut, 1..64 (0 = the
                             library's cut) */
  int32_t decode_depth;   /* QN_KERNEL_DECODE: weight tiles in flight per wave: 0 (the default, 3), 2 or 3;
                             QN_KERNEL_FUSED and _WIDE take 0 or 3; with AUTO, 2 rules those two out */
  int32_t general_rows;   /* QN_KERNEL_GENERAL: row groups per workgroup and waves per workgroup, both 0 (the */
  int32_t general_waves;  /* library's shape) or both > 0 naming a built pair (else QN_ERR_UNSUPPORTED) */
  int32_t elem_store;     /* 0 or 1; many-token kernel: 1 stores outputs element by element instead of in 16-byte
                             pieces through LDS (same values) */
  void* main_begin;       /* both NULL, or two hipEvent_t created with timing (the caller's, not retained): the main */
  void* main_end;         /* streaming kernel is launched by hipExtLaunchKernel, which records them at that launch's
                             own begin and end (a kernel trace's interval; events recorded on the stream around the
                             call would also take in the dispatch). Events created with hipEventDisableSystemFence
                             leave out the system-scope release the end event otherwise adds to the kernel.
                             Measurement only: the results are the same. A call with several main launches (token
                             blocks, sub-calls) leaves the last one's. One NULL and one not: QN_ERR_VALUE */
} qn_linear_opts;

/* Workspace bytes of nvfp4_lora_linear_opts with these options (host, pure); 0 if the options are invalid or name
 * a kernel that cannot serve the call. NULL opts = nvfp4_lora_linear_workspace. */
size_t nvfp4_lora_linear_workspace_opts(int64_t m, int64_t k, const qn_proj* projs, int32_t nproj,
                                        const qn_linear_opts* opts);

/* nvfp4_lora_linear with explicit options (NULL = defaults, identical to nvfp4_lora_linear). Errors besides those of
 * nvfp4_lora_linear: QN_ERR_VALUE for an option out of range, QN_ERR_UNSUPPORTED when the named kernel or shape cannot
 * serve the call; in both cases nothing is launched. */
qn_status nvfp4_lora_linear_opts(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                                 const qn_proj* projs, int32_t nproj, int32_t epilogue, const qn_linear_opts* opts,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* nvfp4_lora_linear for callers that cannot allocate memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and kernels, with the scratch space taken from a device
 * array inside the library instead of a caller's workspace. It calls no allocator. The array holds
 * nvfp4_lora_linear_noalloc_max_bytes() bytes (32 MiB) on each GPU the library runs on, for as long as the process
 * lives; it serves every decode-sized call of the configurations here (up to 128 tokens at the 7B and 32B shapes).
 * A call needing more (nvfp4_lora_linear_workspace above the maximum) returns QN_ERR_WORKSPACE and launches nothing.
 * Every call on one GPU shares that GPU's array, so calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race; calls ordered on one stream are safe. The array keeps the last call's
 * contents; it starts zeroed (static device memory) and every call leaves its control words zero, as the workspace
 * contract above asks. Errors: as nvfp4_lora_linear, plus QN_ERR_HIP if the array's
 * device address cannot be looked up. */
qn_status nvfp4_lora_linear_noalloc(const uint16_t* x, int64_t m, int64_t k, int64_t ldx, const qn_aqn* aqn,
                                    const qn_proj* projs, int32_t nproj, int32_t epilogue, void* stream);

/* Bytes of the scratch array behind nvfp4_lora_linear_noalloc (host, pure). */
size_t nvfp4_lora_linear_noalloc_max_bytes(void);

/* Backward of nvfp4_lora_linear (one projection, no norm) through the frozen NVFP4 weight [review §2.1: the backbone is
 * frozen and the gradients update A and B, but may pass through the frozen projection to reach an earlier adapter;
 * §6, steps 8-10]. For y = s_g W_hat h + lambda B (A h) and the upstream gradient g = dL/dy:
 *   dh = s_g W_hat^T g + lambda A^T (B^T g)       [m][lddh], bf16 or f32 (dh_dtype), NULL = not computed
 *   d_a = lambda (B^T g)^T h                      [r][k] f32 row-major, NULL = not computed
 *   d_b = lambda g^T (A h)                        [n][r] f32 row-major, NULL = not computed
 * g [m][ldg] bf16 and h [m][ldh] bf16 (the forward's input; needed for d_a and d_b), 2-byte aligned (16-byte aligned
 * rows are read 16 bytes at a time); the weight in QN_LAYOUT_TILED as for the forward; lora_a [r][k], lora_b [n][r] bf16 (r <= 64; r == 0: no
 * adapter, only dh). bf16 MFMAs with f32 accumulation; the rank-r intermediates are kept in f32 and enter the MFMAs as
 * bf16 hi + lo parts. The weight is read transposed from the tiled layout (dequantized exactly to bf16 in LDS).
 * Results do not depend on scheduling (fixed summation orders). Workspace: nvfp4_lora_linear_backward_workspace
 * (256-byte aligned; none needed when r == 0). Errors: QN_ERR_SHAPE, QN_ERR_ALIGN, QN_ERR_NULL, QN_ERR_VALUE (bad
 * dh_dtype, non-finite lambda), QN_ERR_WORKSPACE, QN_ERR_UNSUPPORTED (r > 64); nothing is launched on an error. */
qn_status nvfp4_lora_linear_backward(const uint16_t* g, int64_t m, int64_t n, int64_t ldg, const uint16_t* h, int64_t k,
                                     int64_t ldh, const uint8_t* codes, const uint8_t* block_scales,
                                     const float* tensor_scale, const uint16_t* lora_a, const uint16_t* lora_b,
                                     int32_t r, float lambda, void* dh, int32_t dh_dtype, int64_t lddh, float* d_a,
                                     float* d_b, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of nvfp4_lora_linear_backward (host, pure). */
size_t nvfp4_lora_linear_backward_workspace(int64_t m, int64_t n, int64_t k, int32_t r);

/* Exponential AQN noise schedule [review §5.2]: sigma_0 = 0, sigma_k = start * (end/start)^((k-1)/8), k = 1..9
 * (stages beyond 9 continue the same geometric decay). Host, pure, fp64. */
double aqn_sigma(int32_t stage, double sigma_start, double sigma_end);

/* Group-relative advantages [review §2.2]: A_i = (R_i - mean) / (pop_std + eps) over each group of g consecutive
 * rewards. rewards, adv: [groups][g] f32 (device); fp64 arithmetic on the device, rounded to f32. */
qn_status grpo_group_advantage(const float* rewards, int32_t groups, int32_t g, float eps, float* adv, void* stream);

/* Measurement helper, not part of the method: reads [src, src + bytes) from device memory once, as a plain streaming
 * kernel (16-byte non-temporal loads, 2048 workgroups of 256 threads), and XORs what it read into *sink (device, the
 * caller zeroes it), so that the rate a memory-bound kernel reaches can be compared with the rate plain streaming
 * reads reach on the same device. bytes % 16 == 0 (QN_ERR_SHAPE), src 16-byte and sink 4-byte aligned (QN_ERR_ALIGN). */
qn_status qn_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Statistics of one grpo_clipped_surrogate call (device struct, written by the call). */
typedef struct {
  double loss;       /* -(sum over valid tokens of w * surrogate), w as set by `agg` */
  double ratio_mean; /* mean token ratio over valid tokens (0 if none) */
  float ratio_min, ratio_max;
  int64_t tokens;    /* valid tokens */
  int64_t clipped;   /* tokens whose clipped term is strictly the smaller (their gradient is zero) */
} qn_grpo_stats;

/* GRPO token ratio and clipped surrogate [review §2.3]: for token t of response i (sampled by the behavior policy),
 *   rho = exp(logp[i][t] - logp_old[i][t]),  s = min(rho A_i, clip(rho, 1 - clip_low, 1 + clip_high) A_i),
 * with A_i the response's group-relative advantage (grpo_group_advantage). loss = -(sum w s) with w = 1 / (valid
 * tokens of the batch) (agg 0) or w = 1 / (responses with tokens x tokens of response i) (agg 1). The pages fix
 * neither the widths nor the combination; both are arguments here. Per token (optional outputs, [n_seq][ld] f32, 0 past
 * the response's length): the surrogate and grad = d loss / d logp = -w rho A where the unclipped term is the smaller
 * (ties included), else 0.
 *   logp, logp_old [n_seq][ld] f32; lengths [n_seq] int32 (valid tokens, clamped to [0, t_max]); adv [n_seq] f32; all
 *   device. fp64 arithmetic from the f32 inputs; one workgroup, statistics summed in a fixed order (deterministic).
 * Errors: QN_ERR_SHAPE (negative sizes, ld < t_max with n_seq > 0), QN_ERR_VALUE (clip_low outside [0, 1), clip_high < 0, bad agg,
 * non-finite widths), QN_ERR_NULL. */
qn_status grpo_clipped_surrogate(const float* logp, const float* logp_old, int64_t ld, const int32_t* lengths,
                                 const float* adv, int32_t n_seq, int32_t t_max, float clip_low, float clip_high,
                                 int32_t agg, float* surrogate, float* grad, qn_grpo_stats* stats, void* stream);

/* Static description of a status code (host). */
const char* qn_status_string(qn_status s);

#ifdef __cplusplus
}
#endif
#endif /* QERL_NVFP4_H */

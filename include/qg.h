/*
 * qg.h -- C ABI of the MI355X (gfx950) quantized GEMM library (libqg.so).
 *
 * What it computes: Y = X . dequant(Wq, scales, zeros)^T with low-bit weights
 * (int4 / uint4 + zero points, FP4 e2m1 with UE8M0 block scales, FP8 e4m3 with
 * channel scales) and f16 / bf16 / FP8 e4m3 activations, as a dense layer and as
 * an MoE grouped GEMM over routed tokens.  Sources: the web pages on the Humming
 * quantized-GEMM library -- "Humming" (README), "Key Features" and "Support Matrix"
 * (weight, activation and scale types; dense and MoE GEMM); "Humming: Fast,
 * Flexible Kernels for Quantized Inference" (the standard format of weights,
 * scales and zero points; preprocessing that repacks tensors into the kernel's
 * layout); "Humming" (wiki article), "Quantization representation", "Kernel
 * configuration and compilation" and "Device and workload selection" (channel /
 * group / block scales, arch-tied transformed layouts, M-range dispatch, the
 * indexed MoE path).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers unless stated otherwise; descriptors and
 *   handles are HOST structs.  The caller owns every allocation; the library never
 *   allocates or frees device memory.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *   call only enqueues work on that stream and returns; there is no host
 *   synchronisation on any path (MoE grids are sized from capacity, not counts).
 * - Arguments are validated on the host BEFORE anything is launched.  On error
 *   nothing is written and the status says why; the library never prints (unless
 *   the environment variable QG_LOG=1) and never throws across the ABI.
 * - QG_ERR_HIP is returned when a launch reports an error (hipGetLastError).
 * - M == 0 (or T == 0) is a successful no-op.
 * - Row-major tensors with contiguous rows; every pointer must be 16-byte aligned.
 * - Workspaces: when qg_workspace_bytes() is non-zero the caller passes a device
 *   buffer of at least that size; its contents need no initialisation (a call writes
 *   every byte it reads).  Calls that share one workspace must not run concurrently
 *   (use one per stream).
 * - Shape rules: n % 64 == 0, k % 128 == 0, k % group_k == 0.
 */
#ifndef QG_H_
#define QG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QG_OK = 0,
  QG_ERR_INVALID_ARG = 1,    /* null / misaligned pointer, negative size, bad enum value      */
  QG_ERR_UNSUPPORTED = 2,    /* valid but unsupported type combination or shape               */
  QG_ERR_ARCH_MISMATCH = 3,  /* prepared for another GPU architecture than the current device */
  QG_ERR_NOT_PREPARED = 4,   /* handle not filled by qg_prepare (magic / layout version)      */
  QG_ERR_WORKSPACE = 5,      /* workspace or output buffer too small                           */
  QG_ERR_CAPACITY = 6,       /* MoE align buffers smaller than the worst-case capacity         */
  QG_ERR_HIP = 7             /* a HIP call or kernel launch failed                             */
} qg_status;

/* Weight storage types (logical layouts are those accepted by qg_prepare). */
enum { QG_W_INT4 = 1,      /* symmetric int4 in [-8, 7], two's-complement nibbles            */
       QG_W_UINT4 = 2,     /* uint4 in [0, 15]; with has_zero, value (u - z) * s              */
       QG_W_FP4_E2M1 = 3,  /* OCP FP4 e2m1 codes                                              */
       QG_W_FP8_E4M3 = 4   /* OCP FP8 e4m3 ("fn") codes                                       */ };
/* Scale types. */
enum { QG_S_F16 = 1, QG_S_BF16 = 2, QG_S_F32 = 3, QG_S_UE8M0 = 4 };
/* Activation types.  FP8 activations come with one float32 scale per row (token); FP4
 * activations (MXFP4: packed e2m1 codes, even K in the low nibble) with one UE8M0 exponent
 * byte per 32 consecutive K of a row. */
enum { QG_A_F16 = 1, QG_A_BF16 = 2, QG_A_FP8_E4M3 = 3, QG_A_FP4_E2M1 = 4 };
/* Output types. */
enum { QG_O_F16 = 1, QG_O_BF16 = 2 };
/* Compute options. */
enum { QG_C_NATIVE = 0,    /* multiply in the activation's type                               */
       QG_C_W_TO_FP8 = 1,  /* int4 weights converted to e4m3 in-kernel (FP8 activations)      */
       /* Flag, OR-ed into either option: batch-invariant execution ("Humming" wiki article,
        * "Precision and deployment considerations": no Stream-K-style split and the same
        * MMA type across batch sizes).  Every row count then runs the MFMA kernel without a
        * split over K, so each output row is bitwise the same whatever M (or T) and the other
        * rows are; slower at small M.  MoE block sizes below 128 are rejected. */
       QG_C_BATCH_INVARIANT = 4 };

/*
 * Layer description ("Layer config": shapes, data types, quantization parameters).
 * Supported combinations (anything else -> QG_ERR_UNSUPPORTED):
 *   int4 / uint4(+zeros) weights, f16|bf16 scales, group_k a multiple of 128 or 0
 *       (per channel), f16|bf16 activations                          [W4A16]
 *   int4 weights, QG_C_W_TO_FP8, bf16|f16 scales (group a multiple of 128, or 0 =
 *       per channel), e4m3 activations                                 [W4A8]
 *   e2m1 weights, UE8M0 scales, group_k == 32, f16|bf16 activations  [MXFP4 W4A16]
 *   e2m1 weights, UE8M0 scales, group_k == 32, e4m3 activations      [MXFP4 W4A8]
 *   e2m1 weights, UE8M0 scales, group_k == 32, e2m1 activations with UE8M0 exponents per
 *       32 K ("Humming" README, "Key Features": FP4 activations)    [MXFP4 W4A4]
 *   e4m3 weights, f32 channel scales (group_k == 0), e4m3 activations [W8A8]
 *   e4m3 weights, f32 block scales (group_k == 128: one scale per 128 output channels x
 *       128 K, scales [E][N/128][K/128], n % 128 == 0), e4m3 activations with one f32
 *       scale per (row, 128-wide K group)                              [block-scaled W8A8]
 */
typedef struct {
  int32_t w_type;       /* QG_W_*                                                      */
  int32_t s_type;       /* QG_S_*                                                      */
  int32_t group_k;      /* elements per scale along K; 0 = one scale per output channel */
  int32_t has_zero;     /* 1: uint4 zero point per (n, group), only with QG_W_UINT4    */
  int32_t a_type;       /* QG_A_*                                                      */
  int32_t compute;      /* QG_C_NATIVE or QG_C_W_TO_FP8, optionally | QG_C_BATCH_INVARIANT */
  int32_t out_type;     /* QG_O_*                                                      */
  int32_t num_experts;  /* 1 for a dense layer                                         */
  int64_t n;            /* output features                                             */
  int64_t k;            /* reduction dimension                                         */
} qg_layer_desc;

/*
 * Prepared-layer handle: a caller-owned host POD filled by qg_prepare.  It records
 * the target architecture (the prepared layout is tied to it) and where the
 * weight, scale and zero regions live inside the caller's device buffer.
 */
typedef struct {
  uint32_t magic;            /* 'QGP1' once prepared                                */
  uint32_t layout_version;   /* 1                                                   */
  uint32_t gfx_arch;         /* 950 for gfx950                                      */
  uint32_t reserved;
  qg_layer_desc desc;
  void* dev;                 /* device buffer holding the prepared image            */
  uint64_t bytes;            /* size of that image                                  */
  uint64_t off_w, off_s, off_z;                 /* region offsets in bytes           */
  uint64_t w_expert_bytes, s_expert_bytes, z_expert_bytes;  /* per-expert strides    */
} qg_prepared;

#define QG_PREPARED_MAGIC 0x31504751u   /* "QGP1" little-endian */
#define QG_LAYOUT_VERSION 1u

/*
 * qg_prepared_bytes: device bytes qg_prepare needs for `desc`; 0 if the
 * description is invalid or unsupported.  Host-only, never touches the GPU.
 */
size_t qg_prepared_bytes(const qg_layer_desc* desc);

/*
 * qg_prepare: the offline transform of a layer.  "Humming: Fast, Flexible Kernels for
 * Quantized Inference", standard-format paragraph: weights, scales and zero points stay
 * separate parameters, and a preprocessing step checks them, pads and reorders them into
 * the layout the kernel reads.  "Humming" (wiki article), "Quantization representation":
 * the transform runs before the first forward call and its result belongs to one GPU
 * architecture (here: gfx_arch, checked by every later call).  "Humming" (wiki article),
 * "Kernel configuration and compilation": one stored layout serves every compute and
 * tuning choice made per call, so one prepared image serves every M and every tile.
 *   w      device, logical weights of all experts, contiguous:
 *            int4/uint4  uint32 [E][N][K/8]  (element k at bits 4*(k%8), low nibble first)
 *            e2m1        uint8  [E][N][K/2]  (even k in the low nibble)
 *            e4m3        uint8  [E][N][K]
 *   scales device, [E][N][G] of the scale type (G = K/group_k, or 1 per channel);
 *          block-scaled e4m3: float32 [E][N/128][K/128]
 *   zeros  device, uint8 [E][N][G] holding 0..15 when has_zero, else NULL
 *   Every byte of the prepared image is written (alignment padding as zeros).
 *   dev_out device buffer of at least qg_prepared_bytes(desc) bytes (must not
 *          overlap the inputs); `out` (host) receives the handle.
 * Enqueued on `stream`; the inputs may be freed once the stream has passed it.
 */
qg_status qg_prepare(const qg_layer_desc* desc, const void* w, const void* scales, const void* zeros,
                     void* dev_out, size_t dev_bytes, qg_prepared* out, void* stream);

/*
 * qg_workspace_bytes: device workspace qg_gemm / qg_moe_gemm need for m rows
 * (dense) or T tokens x topk (MoE; pass topk = 0 for dense).  0 means none.
 * "Humming" (wiki article), "Device and workload selection": the configuration,
 * including a split of the reduction, is chosen per range of M; "Precision and
 * deployment considerations": a Stream-K-style split is a tuning control.  The
 * workspace holds what such a split (or the W4A8 route below, this library's own
 * reading) needs between launches.
 *   - dense shapes whose output tiles fill at most half the GPU split K over
 *     workgroups: ksplit * m * N * 4 bytes of fp32 partial sums (required:
 *     QG_ERR_WORKSPACE without it);
 *   - grouped (MoE) products need none.
 */
size_t qg_workspace_bytes(const qg_prepared* p, int64_t m_or_tokens, int32_t topk);

/*
 * qg_gemm: dense Y[m, n] = sum_k X[m, k] * W[n, k] for a prepared dense layer.
 * "Humming" (README), "Usage Example": the quantized layer applied to inputs gives the
 * product of the inputs with the transposed (dequantized) weight.  "Humming" (wiki
 * article), "Device and workload selection": the kernel configuration follows the range
 * of M, switching where compute starts to outweigh the weight traffic.
 *   x        device [M][K] of a_type (f16/bf16 values or e4m3 codes), or packed e2m1 codes
 *            uint8 [M][K/2] for FP4 activations
 *   x_scale  device, else NULL: float32 per-token scales for e4m3 activations, [M], or
 *            [M][K/128] for block-scaled layers; uint8 UE8M0 exponents [M][K/32] for FP4
 *            activations (X[m, k] = e2m1(code) * 2^(x_scale[m][k/32] - 127))
 *   y        device [M][N] of out_type, written in full (fp32 accumulation, RNE)
 *   ws       device workspace of ws_bytes >= qg_workspace_bytes(p, m, 0)
 * The tile / split-K choice is made from M on the host (the M-bucket selector).
 */
qg_status qg_gemm(const qg_prepared* p, const void* x, const void* x_scale, void* y, int64_t m,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * qg_gemm_noalloc: for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The same product,
 * kernels and tile / split choice as qg_gemm(p, x, x_scale, y, m, ws, ws_bytes, stream),
 * with the workspace taken from a device array of this library holding
 * qg_noalloc_scratch_bytes() = 32 MiB, one per GPU, kept until the process ends.  No call
 * allocates or frees memory.  Every dense split over K the selector makes fits (at most
 * 32 MiB of partials); a workspace beyond the array would be QG_ERR_WORKSPACE before any
 * launch.  Nothing in the array must start at zero: each call writes what it reads.  All calls on one GPU share its array, so calls that overlap on that GPU
 * (concurrent streams, or host threads) race and give wrong results: serialise them.
 */
qg_status qg_gemm_noalloc(const qg_prepared* p, const void* x, const void* x_scale, void* y, int64_t m,
                          void* stream);
size_t qg_noalloc_scratch_bytes(void);

/*
 * MoE routing preparation (the indexed input path: rows are gathered through
 * routing indices).  qg_moe_block_m returns the row-block size the grouped GEMM
 * will use for T tokens with topk slots (0 on an invalid handle).
 * qg_moe_capacity returns the worst-case buffer sizes for any routing:
 *   cap_sorted = roundup(T*topk + min(E, T*topk)*(block_m - 1), block_m),
 *   cap_blocks = cap_sorted / block_m.
 */
int32_t qg_moe_block_m(const qg_prepared* p, int64_t tokens, int32_t topk);
qg_status qg_moe_capacity(int64_t tokens, int32_t topk, int32_t num_experts, int32_t block_m,
                          int64_t* cap_sorted, int64_t* cap_blocks);

/*
 * qg_moe_align: token-to-expert sort and padding for the indexed MoE organization
 * ("Humming" wiki article, "Device and workload selection").  The pages give no
 * algorithm for it; the contract below (stable order, sentinel, padding) is this
 * library's.
 *   topk_ids   device int32 [T][topk]; flat index f = t*topk + j; ids outside [0, E) are dropped
 *   sorted_ids device int32 [cap_sorted]: for each expert e in ascending order, the flat
 *              indices routed to e in ascending order, padded with the sentinel T*topk to a
 *              multiple of block_m; sentinel after the end
 *   expert_ids device int32 [cap_blocks]: expert of each block_m-row block, -1 after the end
 *   num_post_pad device int32 [1]: total padded rows
 * Deterministic: the result is unique and bit-exact.  Capacities below
 * qg_moe_capacity -> QG_ERR_CAPACITY.  block_m must be a power of two in [1, 256].
 */
qg_status qg_moe_align(const int32_t* topk_ids, int64_t tokens, int32_t topk, int32_t num_experts,
                       int32_t block_m, int32_t* sorted_ids, int64_t cap_sorted, int32_t* expert_ids,
                       int64_t cap_blocks, int32_t* num_post_pad, void* stream);

/*
 * The grouped MoE input organizations ("Humming" wiki article, "Device and workload
 * selection": grouped-contiguous execution keeps each expert's rows together;
 * grouped-masked execution gives each expert its own storage with a count of valid rows).
 * Both name input rows directly: qg_moe_grouped_map writes the block map in qg_moe_align's
 * contract (rows of each expert in ascending order, padded to block_m with the sentinel
 * rows_total; the expert of every block; the padded total), after which
 *     qg_moe_gemm(p, x, x_scale, sorted_ids, expert_ids, num_post_pad,
 *                 rows_total, 1, block_m, y, ws, ws_bytes, stream)
 * computes y[r] = x[r] . W_e^T for every row r of expert e; y has x's row layout and rows
 * that belong to no expert are not written.
 *   layout = QG_MOE_CONTIGUOUS: offsets_or_counts = device int32 [E+1], expert e owns rows
 *            [offsets[e], offsets[e+1]) of x [rows_total][K]; offsets[0] = 0, non-decreasing,
 *            offsets[E] <= rows_total (offsets are clamped to [0, rows_total] and made
 *            non-decreasing on the device, so malformed offsets give a wrong map, never an
 *            out-of-range write); rows_per_expert is ignored.
 *   layout = QG_MOE_MASKED: offsets_or_counts = device int32 [E] valid-row counts (clamped to
 *            [0, rows_per_expert]); x is [E][rows_per_expert][K] = [rows_total][K] with
 *            rows_total = E * rows_per_expert (else QG_ERR_INVALID_ARG).
 * Buffers as for qg_moe_align with capacities qg_moe_capacity(rows_total, 1, E, block_m)
 * (QG_ERR_CAPACITY below them); block_m a power of two in [1, 256] (the GEMM then takes the
 * block sizes qg_moe_gemm lists; qg_moe_block_m(p, rows, 1) picks one for about `rows`
 * valid rows).  E <= 1024, rows_total <= 2^30.
 */
enum { QG_MOE_CONTIGUOUS = 1, QG_MOE_MASKED = 2 };
qg_status qg_moe_grouped_map(int32_t layout, const int32_t* offsets_or_counts, int32_t num_experts,
                             int64_t rows_total, int64_t rows_per_expert, int32_t block_m, int32_t* sorted_ids,
                             int64_t cap_sorted, int32_t* expert_ids, int64_t cap_blocks, int32_t* num_post_pad,
                             void* stream);

/*
 * qg_moe_gemm: grouped GEMM over the aligned rows.  For every (token t, slot j)
 * with e = topk_ids[t][j] in [0, E):  Y[t*topk + j, :] = X[t] . W_e^T.
 * "Humming" (wiki article), "Quantization representation": MoE weights carry an expert
 * dimension; "Device and workload selection": in the indexed organization the kernel
 * reads each expert's input rows through the routing indices (here sorted_ids).
 *   x        device [T][K] of a_type (FP4: uint8 [T][K/2]);  x_scale device float32 [T] for
 *            e4m3 ([T][K/128] for block-scaled layers), uint8 [T][K/32] for FP4, else NULL
 *   sorted_ids / expert_ids / num_post_pad  from qg_moe_align with the same block_m
 *   block_m  4, 16, 32 or 64 (weight-streaming kernel) or 128, 256 (MFMA kernel; 256 not
 *            for e4m3 or int4->e4m3 weights); FP4 activations: 16, 32, 64 or 128;
 *            qg_moe_block_m picks one, any other is QG_ERR_UNSUPPORTED
 *   y        device [T*topk][N] of out_type; rows of dropped slots are not written
 * The grid is sized from capacity; blocks past num_post_pad exit at once.
 */
qg_status qg_moe_gemm(const qg_prepared* p, const void* x, const void* x_scale, const int32_t* sorted_ids,
                      const int32_t* expert_ids, const int32_t* num_post_pad, int64_t tokens, int32_t topk,
                      int32_t block_m, void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * The rest of an MoE layer.  The pages time an MoE layer as the sum of its gate/up and
 * down grouped products ("Humming: Fast, Flexible Kernels for Quantized Inference",
 * benchmark paragraph; "Humming" wiki article, "Reported performance") and do not say
 * what joins them; this library's reading is the usual SwiGLU feed-forward layer:
 *
 *   1. qg_moe_align, then qg_moe_gemm with the gate/up layer (N = 2*I): Y1 [T*topk][2I];
 *   2. qg_moe_swiglu: act = silu(gate) * up per (token, slot) row -> [T*topk][I];
 *   3. the down product is qg_moe_gemm itself with the down layer (K = I), called with
 *      tokens = T*topk and topk = 1 on the SAME align output: flat index f then names input
 *      row f of act, the sentinel T*topk is unchanged, and Y2[f] = act[f] . W_e^T; its
 *      block_m is qg_moe_block_m(p_down, T*topk, 1), which must equal the align's block_m
 *      (it does when both layers use the same kernel family; else align again);
 *   4. qg_moe_combine: out[t] = sum_j w[t][j] * Y2[t*topk + j] over routed slots.
 */

/*
 * qg_moe_swiglu: act[r][i] = silu(g) * u with g = gate_up[r][i], u = gate_up[r][inter + i],
 * silu(g) = g / (1 + e^-g), computed in float32, for every row r < rows.
 *   gate_up   device [rows][2*inter], in_type QG_O_F16 or QG_O_BF16 (the gate/up output type)
 *   out_type  QG_A_F16 / QG_A_BF16: act rounded to nearest even, written to out [rows][inter];
 *             QG_A_FP8_E4M3: each row quantized for the next product's FP8 activations:
 *             out_scale[r] = max_i |act[r][i]| / 448 (float32; 1 for an all-zero row) and
 *             out (uint8 [rows][inter]) = e4m3 codes, round to nearest even of
 *             clamp(act / out_scale[r], -448, 448)
 *             QG_A_FP4_E2M1: each row quantized for the next product's MXFP4 activations: act
 *             rounded to bfloat16 (nearest even), then exactly qg_quantize_e2m1_rows of those
 *             rows; out = packed e2m1 codes uint8 [rows][inter/2] (16-byte aligned)
 *   out_scale device float32 [rows] for QG_A_FP8_E4M3, uint8 [rows][inter/32] UE8M0 exponents
 *             for QG_A_FP4_E2M1, else ignored (may be NULL)
 * inter % 8 == 0 (and inter <= 8192 for QG_A_FP8_E4M3, inter % 32 == 0 for QG_A_FP4_E2M1),
 * else QG_ERR_UNSUPPORTED.  Rows of
 * slots the gate/up product did not write give unspecified values, which nothing reads.
 */
qg_status qg_moe_swiglu(const void* gate_up, int64_t rows, int64_t inter, int32_t in_type, int32_t out_type,
                        void* out, void* out_scale, void* stream);

/*
 * qg_quantize_e4m3_rows: per-token FP8 quantization of 16-bit activations, the input of the
 * W4A8 and W8A8 products ("Humming" wiki article, "Reported performance": tokenwise FP8
 * activations).  For each row r < rows of x (device [rows][k], in_type QG_A_F16 / QG_A_BF16):
 *   scale[r] = max_i |x[r][i]| / 448 in float32 (1 for an all-zero row),
 *   codes[r][i] = e4m3 code, round to nearest even, of clamp(x[r][i] / scale[r], -448, 448).
 *   codes  device uint8 [rows][k] (8-byte aligned);  scale  device float32 [rows]
 * k % 8 == 0 and k <= 8192, else QG_ERR_UNSUPPORTED.
 */
qg_status qg_quantize_e4m3_rows(const void* x, int64_t rows, int64_t k, int32_t in_type, uint8_t* codes, float* scale,
                                void* stream);

/*
 * qg_quantize_e2m1_rows: MXFP4 quantization of 16-bit activations, the input of the W4A4
 * products ("Humming" README, "Key Features": FP4 activations and UE8M0 scales).  The pages
 * give no rule; this is the OCP Microscaling v1.0 conversion.  For each block of 32
 * consecutive elements of a row of x (device [rows][k], in_type QG_A_F16 / QG_A_BF16, finite):
 *   E = floor(log2(max |block|)) - 2, clamped to [-127, 127] (-127 for an all-zero block),
 *   scales[r][b] = E + 127 (UE8M0);
 *   each element's code = the e2m1 value nearest to x / 2^E, ties to the even code, values
 *   above 6 in magnitude give 6; negative codes only for non-zero magnitudes.
 *   codes  device uint8 [rows][k/2], 16-byte aligned (even k in the low nibble)
 *   scales device uint8 [rows][k/32]
 * k % 32 == 0, else QG_ERR_UNSUPPORTED.
 */
qg_status qg_quantize_e2m1_rows(const void* x, int64_t rows, int64_t k, int32_t in_type, uint8_t* codes,
                                uint8_t* scales, void* stream);

/*
 * qg_moe_combine: out[t][:] = sum over slots j with 0 <= topk_ids[t][j] < E of
 * weights[t][j] * y[t*topk + j][:], accumulated in float32 in slot order and rounded once
 * (nearest even).  Rows of other slots may be read but never contribute (they may hold
 * anything, NaN included).
 *   y         device [T*topk][n] of dtype (QG_O_F16 / QG_O_BF16), e.g. the down product's output
 *   weights   device float32 [T][topk] (the router's probabilities; applied as given)
 *   topk_ids  device int32 [T][topk]
 *   out       device [T][n] of dtype, written in full
 * n % 8 == 0, else QG_ERR_UNSUPPORTED.  Tokens with no routed slot get zeros.
 */
qg_status qg_moe_combine(const void* y, const float* weights, const int32_t* topk_ids, int64_t tokens, int32_t topk,
                         int32_t num_experts, int64_t n, int32_t dtype, void* out, void* stream);

/*
 * qg_dequant: writes expert `expert` of a prepared layer back as dense float32
 * [N][K] = code value (minus zero point) times scale, read through the same
 * unpack routines the GEMM kernels use.  Every such value is exact in float32
 * except e4m3 x f32 channel scale, which is one correctly rounded product.
 * Block-scaled e4m3 layers: QG_ERR_UNSUPPORTED (their image is checked byte for byte).
 * For checking the prepared layout; not on the GEMM path.
 */
qg_status qg_dequant(const qg_prepared* p, int32_t expert, float* out, void* stream);

/*
 * Measurement helpers (not on the GEMM path): the ceilings a kernel's time is read against.
 * The pages time kernels with a cold L2 ("Humming: Fast, Flexible Kernels for Quantized
 * Inference", benchmark paragraph) and quote rooflines of bandwidth and matrix throughput
 * ("Humming" wiki article, "Device and workload selection"); these measure what this GPU
 * delivers of each.
 *
 * qg_ceiling_read: reads `bytes` of buf once with 16-byte loads, loads_per_lane (1, 2, 4,
 *   8 or 16) per lane, all issued before any is used, in ceil(bytes / (4096 *
 *   loads_per_lane)) workgroups of 256 lanes; writes one word per wave to sink
 *   (device uint32, sink_words >= 4 * workgroups, else QG_ERR_WORKSPACE).
 *   buf device, 16-byte aligned, 0 < bytes < 2^31, bytes % 16 == 0.
 * qg_ceiling_mfma: `workgroups` workgroups of 4 waves, each wave issuing iters x 4
 *   independent MFMAs from registers: dtype 0 = bf16 32x32x16 (32768 flop each), 1 = e4m3
 *   32x32x64 (131072), 2 = e2m1 x e2m1 32x32x64 (131072); sink device float32
 *   [workgroups * 256].
 */
qg_status qg_ceiling_read(const void* buf, uint64_t bytes, int32_t loads_per_lane, uint32_t* sink,
                          uint64_t sink_words, void* stream);
qg_status qg_ceiling_mfma(int32_t dtype, int64_t iters, int32_t workgroups, float* sink, uint64_t sink_floats,
                          void* stream);
/* qg_ceiling_lds: `workgroups` workgroups of 8 waves, each lane reading iters x 8 x 16 bytes
 * of its CU's LDS (64 KiB, conflict-free addresses); sink device uint32 [workgroups * 512]. */
qg_status qg_ceiling_lds(int64_t iters, int32_t workgroups, uint32_t* sink, uint64_t sink_words, void* stream);

/* Human-readable name of a status code (static string). */
const char* qg_status_str(qg_status s);

/* Library / layout version: (major << 16) | minor. */
int32_t qg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QG_H_ */

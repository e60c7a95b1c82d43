// Host side of libqg.so: the C ABI declared in include/qg.h.  Validation happens
// here, before anything is launched; then the M-bucket selector picks a kernel
// family and tile ("Humming" wiki article, "Device and workload selection": ranges of
// M get their own configurations, chosen by where computation starts to dominate
// weight transfer) and the launch is enqueued on the caller's stream.
#include <stdio.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "qg.h"
#include "qg_device.h"
#include "qg_kernels.h"

using namespace qg;

namespace {

bool log_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("QG_LOG");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

#define QG_LOG(...)                         \
  do {                                      \
    if (log_enabled()) {                    \
      fprintf(stderr, "[qg] " __VA_ARGS__); \
      fputc('\n', stderr);                  \
    }                                       \
  } while (0)

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Architecture of the current device: 950 for gfx950, 0 if unknown, -1 on error.
int current_arch() {
  static std::mutex mu;
  static int cached[64];
  static bool init[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  std::lock_guard<std::mutex> lk(mu);
  if (dev < 64 && init[dev]) return cached[dev];
  hipDeviceProp_t prop;
  int arch = -1;
  if (hipGetDeviceProperties(&prop, dev) == hipSuccess) arch = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 950 : 0;
  if (dev < 64) { cached[dev] = arch; init[dev] = true; }
  return arch;
}

// Which kernel weight path a layer uses.
struct PathInfo {
  int wp_small;   // path of the weight-streaming kernel
  int wp_mfma;    // path of the MFMA-bound kernel
  int order;      // repack nibble order: 0 natural, 1 pair, 2 quad
  int bias8;      // repack stores q + 8
  int w4;         // 4-bit codes
  int af, of, st;
  int dq_wp;      // path used for the read-back check
  int binv;       // batch-invariant: MFMA kernel for every row count, no split over K
};

int scale_bytes(int s_type) {
  switch (s_type) {
    case QG_S_F16: case QG_S_BF16: return 2;
    case QG_S_F32: return 4;
    case QG_S_UE8M0: return 1;
    default: return 0;
  }
}

// Host-only validation of a layer description.
qg_status check_desc(const qg_layer_desc* dd, PathInfo* pi) {
  if (!dd) return QG_ERR_INVALID_ARG;
  // the batch-invariant flag only steers the selector; validate the rest without it
  qg_layer_desc dv = *dd;
  const int binv = (dv.compute & QG_C_BATCH_INVARIANT) != 0;
  dv.compute &= ~QG_C_BATCH_INVARIANT;
  const qg_layer_desc* d = &dv;
  if (d->w_type < QG_W_INT4 || d->w_type > QG_W_FP8_E4M3) return QG_ERR_INVALID_ARG;
  if (d->s_type < QG_S_F16 || d->s_type > QG_S_UE8M0) return QG_ERR_INVALID_ARG;
  if (d->a_type < QG_A_F16 || d->a_type > QG_A_FP4_E2M1) return QG_ERR_INVALID_ARG;
  if (d->out_type != QG_O_F16 && d->out_type != QG_O_BF16) return QG_ERR_INVALID_ARG;
  if (d->compute != QG_C_NATIVE && d->compute != QG_C_W_TO_FP8) return QG_ERR_INVALID_ARG;
  if (d->has_zero != 0 && d->has_zero != 1) return QG_ERR_INVALID_ARG;
  if (d->n <= 0 || d->k <= 0 || d->num_experts <= 0 || d->group_k < 0) return QG_ERR_INVALID_ARG;
  if (d->n % 64 != 0 || d->k % 128 != 0) return QG_ERR_UNSUPPORTED;
  if (d->n > (1 << 30) || d->k > (1 << 20) || d->num_experts > 4096) return QG_ERR_UNSUPPORTED;
  if (d->group_k != 0 && d->k % d->group_k != 0) return QG_ERR_UNSUPPORTED;
  PathInfo p{};
  p.of = d->out_type == QG_O_F16 ? O_F16 : O_BF16;
  const bool act16 = d->a_type == QG_A_F16 || d->a_type == QG_A_BF16;
  if (d->w_type == QG_W_INT4 || d->w_type == QG_W_UINT4) {
    if (d->w_type == QG_W_UINT4 && !d->has_zero) return QG_ERR_UNSUPPORTED;
    if (d->w_type == QG_W_INT4 && d->has_zero) return QG_ERR_UNSUPPORTED;
    if (d->group_k != 0 && d->group_k % 128 != 0) return QG_ERR_UNSUPPORTED;
    if (d->s_type != QG_S_F16 && d->s_type != QG_S_BF16) return QG_ERR_UNSUPPORTED;
    p.w4 = 1;
    if (act16 && d->compute == QG_C_NATIVE) {
      // 16-bit activations: scale and output types follow the activation type
      const int t = d->a_type == QG_A_F16 ? QG_S_F16 : QG_S_BF16;
      if (d->s_type != t || d->out_type != (d->a_type == QG_A_F16 ? QG_O_F16 : QG_O_BF16)) return QG_ERR_UNSUPPORTED;
      p.wp_small = WP_INT4_MAGIC; p.order = 1; p.bias8 = d->w_type == QG_W_INT4;
      p.af = d->a_type == QG_A_F16 ? A_F16 : A_BF16;
      p.dq_wp = WP_INT4_MAGIC;
    } else if (d->a_type == QG_A_FP8_E4M3 && d->compute == QG_C_W_TO_FP8 && d->w_type == QG_W_INT4) {
      if ((d->s_type == QG_S_BF16) != (d->out_type == QG_O_BF16)) return QG_ERR_UNSUPPORTED;
      p.wp_small = WP_INT4Q_MAGIC; p.order = 2; p.bias8 = 0; p.af = A_FP8;
      p.dq_wp = WP_INT4Q_FP8;
    } else {
      return QG_ERR_UNSUPPORTED;
    }
    p.st = d->s_type == QG_S_F16 ? S_F16 : S_BF16;
  } else if (d->w_type == QG_W_FP4_E2M1) {
    if (d->compute != QG_C_NATIVE || d->has_zero || d->group_k != 32 || d->s_type != QG_S_UE8M0)
      return QG_ERR_UNSUPPORTED;
    if (act16) {
      if (d->out_type != (d->a_type == QG_A_F16 ? QG_O_F16 : QG_O_BF16)) return QG_ERR_UNSUPPORTED;
      p.af = d->a_type == QG_A_F16 ? A_F16 : A_BF16;
    } else if (d->a_type == QG_A_FP4_E2M1) {
      p.af = A_FP4;   // W4A4 MXFP4: both operands and both exponents go to the scaled fp4 MFMA
    } else {
      p.af = A_FP8;   // W4A8 MXFP4: e2m1 codes and UE8M0 scales are operands of the scaled fp8/fp4 MFMA
    }
    p.wp_small = WP_FP4; p.order = 0; p.w4 = 1; p.st = S_UE8M0;
    p.dq_wp = WP_FP4;
  } else {  // e4m3: channel scales (group 0) or 128 x 128 block scales (group 128)
    if (d->a_type != QG_A_FP8_E4M3 || d->compute != QG_C_NATIVE || d->has_zero ||
        (d->group_k != 0 && d->group_k != 128) || d->s_type != QG_S_F32)
      return QG_ERR_UNSUPPORTED;
    if (d->group_k == 128 && d->n % 128 != 0) return QG_ERR_UNSUPPORTED;
    p.wp_small = d->group_k == 128 ? WP_FP8_BLOCK : WP_FP8; p.w4 = 0; p.af = A_FP8; p.st = S_F32;
    p.dq_wp = WP_FP8;
  }
  p.wp_mfma = p.wp_small == WP_INT4Q_MAGIC ? WP_INT4Q_FP8 : p.wp_small;
  p.binv = binv;
  if (pi) *pi = p;
  return QG_OK;
}

struct Sizes { int64_t wb, sb, zb, off_s, off_z, total, groups; };

Sizes sizes_of(const qg_layer_desc* d) {
  Sizes s{};
  const int bits = d->w_type == QG_W_FP8_E4M3 ? 8 : 4;
  s.groups = d->group_k == 0 ? 1 : d->k / d->group_k;
  s.wb = d->n * d->k * bits / 8;                     // per expert
  s.sb = d->n * s.groups * scale_bytes(d->s_type);   // per expert
  if (d->w_type == QG_W_FP8_E4M3 && d->group_k > 0) s.sb = (d->n / d->group_k) * s.groups * 4;   // block scales
  s.zb = d->has_zero ? (d->n / 16) * s.groups * 8 : 0;
  const int64_t e = d->num_experts;
  s.off_s = align256(e * s.wb);
  s.off_z = s.off_s + align256(e * s.sb);
  s.total = s.off_z + align256(e * s.zb);
  return s;
}

qg_status check_prepared(const qg_prepared* p, PathInfo* pi) {
  if (!p) return QG_ERR_INVALID_ARG;
  if (p->magic != QG_PREPARED_MAGIC || p->layout_version != QG_LAYOUT_VERSION) return QG_ERR_NOT_PREPARED;
  qg_status s = check_desc(&p->desc, pi);
  if (s != QG_OK) return QG_ERR_NOT_PREPARED;
  if (!p->dev || p->bytes < (uint64_t)sizes_of(&p->desc).total) return QG_ERR_NOT_PREPARED;
  if (p->gfx_arch != 950) return QG_ERR_ARCH_MISMATCH;
  return QG_OK;
}

qg_status check_arch() {
  const int a = current_arch();
  if (a < 0) return QG_ERR_HIP;
  if (a != 950) return QG_ERR_ARCH_MISMATCH;
  return QG_OK;
}

qg_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    QG_LOG("launch failed: %s", hipGetErrorString(e));
    return QG_ERR_HIP;
  }
  return QG_OK;
}

// ---- M-bucket selector --------------------------------------------------------------
// Weight-streaming family: a workgroup of 2 column blocks x 4 K parts (4-bit weights)
// or 1 x 8 (e4m3 weights) waves; rows in blocks of 4 / 16 / 32 / 64 (mt = 0 / 1 / 2 / 4).
StreamTile stream_tile(int64_t rows, int64_t n, int w_type) {
  StreamTile t{};
  const bool w8 = w_type == QG_W_FP8_E4M3;
  t.ncb = w8 ? 1 : 2;
  t.kq = w8 ? 8 : 4;
  t.mt = rows <= 4 ? 0 : (rows <= 16 ? 1 : (rows <= 32 ? 2 : 4));
  const int64_t bm = t.mt == 0 ? 4 : 16 * t.mt;
  t.grid_x = (unsigned)((n / 16 + t.ncb - 1) / t.ncb);
  t.grid_y = (unsigned)((rows + bm - 1) / bm);
  return t;
}

// MFMA-bound family: rows per tile 256 while that still leaves about 1.5 workgroups per
// CU, else 128 (e4m3 weights always 128).
constexpr int kCUs = 256;
constexpr int64_t kStreamMaxRows = 64;


// Split K over workgroups when 128-row tiles would fill at most half of the CUs (above
// that, writing and re-reading the fp32 partials costs more than the idle CUs):
// the largest power of two (at most 8) that keeps the grid within one workgroup per
// CU, leaves every slice whole scale groups and at least 8 K steps.
constexpr int kMaxSplit = 8;
int split_for(int64_t tiles, int64_t k, int group, const PathInfo& pi) {
  if (pi.binv || tiles * 2 > kCUs) return 1;
  const int64_t bk = pi.af == A_FP8 ? 128 : 64;   // K per step: fp8 MFMAs take 128
  const int64_t steps = k / bk;
  int sp = 1;
  while (sp < kMaxSplit && tiles * sp * 2 <= kCUs && steps % (sp * 2) == 0 && steps / (sp * 2) >= 8 &&
         (group <= 0 || (k / (sp * 2)) % group == 0))
    sp *= 2;
  return sp;
}

// 256-row tiles take about 7/8 of the time of two 128-row tiles (each weight is converted and
// fed once per 256 rows instead of twice); with one workgroup per CU at a time a launch takes as
// many tile times as it has rounds of workgroups, so 256 rows are taken when their rounds cost
// less: dense W4A16 N = K = 8192 at M = 2048 (one round of 256-row tiles against two of 128)
// 249 -> 220 us, W4A8 MXFP4 at M = 3072 (1.5 rounds of 256-row against 3 of 128) keeps 128
// rows, 197 -> 178 us.
bool rows256(int64_t rows, int64_t ntiles) {
  const int64_t r256 = ((rows + 255) / 256 * ntiles + kCUs - 1) / kCUs;
  const int64_t r128 = ((rows + 127) / 128 * ntiles + kCUs - 1) / kCUs;
  return 2 * 7 * r256 < 8 * r128;
}

// Dense tiles (MoE tiles are built by qg_moe_gemm).
MfmaTile mfma_tile(int64_t rows, int64_t n, int64_t k, int group, const PathInfo& pi) {
  MfmaTile t{};
  const int64_t ntiles = (n + 255) / 256;
  t.bm = rows256(rows, ntiles) ? 256 : 128;
  // Few rows: 64-row tiles with K split when the split applies.  Half the rows per tile
  // halve the partial sums written and read back; they double the weight conversion per FLOP,
  // which the byte-operand paths barely have: 64-row tiles up to 64 rows (dense W4A16 8192^2
  // at 33 / 64 rows 25.1 / 27.3 -> 20.1 / 23.7 us, slower at 96 / 128 rows), and up to 128
  // rows for e4m3 and e2m1 x e4m3 weights (W4A8 MXFP4 at 96 / 128 rows 25.6 / 29.8 -> 19.8 /
  // 21.2 us, block-scaled W8A8 27.8 / 29.3 -> 25.3 / 26.4 us).
  const int64_t rows64 = pi.af == A_FP8 && pi.wp_mfma != WP_INT4Q_FP8 ? 128 : 64;
  if (t.bm == 128 && rows <= rows64 && pi.af != A_FP4 && !pi.binv) {
    const int64_t tiles64 = ((rows + 63) / 64) * ntiles;
    const int sp64 = split_for(tiles64, k, group, pi);
    if (sp64 > 1) {
      t.bm = 64;
      t.grid_x = (unsigned)tiles64;
      t.grid_y = 1;
      t.ksplit = sp64;
      return t;
    }
  }
  const int64_t tiles = ((rows + t.bm - 1) / t.bm) * ntiles;
  t.grid_x = (unsigned)tiles;
  t.grid_y = 1;
  t.ksplit = t.bm == 128 ? split_for(tiles, k, group, pi) : 1;
  return t;
}

// Dense weight streaming for 5..32 rows (block-scaled: 64): workgroups of 8 column blocks (128 columns) x 1 K
// part, with K split over up to 8 workgroups so that about one workgroup per CU remains.
// Each workgroup then stages only its slice of K for its rows (one LDS round at 16 rows)
// instead of all of K; the fp32 partials are summed by the split-K reduction.  1..4 rows
// keep the 2 x 4 shape without a split (their 4-row staging is already one round).
// Layers of at most 2^22 weights (2 MiB of 4-bit codes) are launch-bound: they also keep
// the 2 x 4 shape, K parts added inside the workgroup, so the product is one launch
// instead of a split plus the reduction's launch.
constexpr int64_t kTinyWeights = (int64_t)1 << 22;
int stream_split(int64_t rows, int64_t n, int64_t k, int group) {
  if (rows <= 4 || n * k <= kTinyWeights) return 1;
  const int64_t groups = (n / 16 + 7) / 8;
  const int64_t chunks = k / 128;
  int sp = 1;
  while (sp < 8 && groups * sp * 2 <= kCUs && chunks % (sp * 2) == 0 &&
         (group <= 0 || (k / (sp * 2)) % group == 0))
    sp *= 2;
  return sp;
}

// Block-scaled e4m3 above the streaming sizes (and at every size under the batch-invariant
// flag): the MFMA kernel's tiles and K split (its promotion per 128-wide step leaves the split-K
// partials scaled, so their reduction only adds them).
bool is_block(const PathInfo& pi) { return pi.wp_small == WP_FP8_BLOCK; }

// Dense rows up to which the streaming kernel runs: 32, where its 64-row tiles lose to the
// MFMA kernel's 128-row tiles with K split (dense W4A16 N = K = 8192: 40..64 rows 30.6-31.7 us
// streamed, 23.6-25.4 us on the MFMA kernel; e4m3 and e2m1 x e4m3 weights alike, at 32 rows
// and below the streaming kernel is faster), 64 for block-scaled e4m3 (streamed 15-22 us
// against 21-24 us at 17..64 rows).
int64_t dense_stream_max(const PathInfo& pi) { return is_block(pi) ? 64 : 32; }
MfmaTile block_tile(int64_t rows, int64_t n, int64_t k, const PathInfo& pi) { return mfma_tile(rows, n, k, 128, pi); }

// Workspace of a dense call: the split-K partial sums.
size_t dense_workspace(const qg_prepared* p, const PathInfo& pi, int64_t m) {
  if (pi.af == A_FP4) return 0;   // W4A4 splits K only inside a workgroup
  if (is_block(pi) && (m > dense_stream_max(pi) || pi.binv)) {
    const MfmaTile t = block_tile(m, p->desc.n, p->desc.k, pi);
    return t.ksplit > 1 ? (size_t)t.ksplit * (size_t)m * (size_t)p->desc.n * sizeof(float) : 0;
  }
  if (m <= dense_stream_max(pi) && !pi.binv) {
    const int sp = stream_split(m, p->desc.n, p->desc.k, p->desc.group_k);
    return sp > 1 ? (size_t)sp * (size_t)m * (size_t)p->desc.n * sizeof(float) : 0;
  }
  const MfmaTile t = mfma_tile(m, p->desc.n, p->desc.k, p->desc.group_k, pi);
  return t.ksplit > 1 ? (size_t)t.ksplit * (size_t)m * (size_t)p->desc.n * sizeof(float) : 0;
}

}  // namespace

extern "C" {

const char* qg_status_str(qg_status s) {
  switch (s) {
    case QG_OK: return "ok";
    case QG_ERR_INVALID_ARG: return "invalid argument";
    case QG_ERR_UNSUPPORTED: return "unsupported type combination or shape";
    case QG_ERR_ARCH_MISMATCH: return "prepared layout / device architecture mismatch";
    case QG_ERR_NOT_PREPARED: return "handle not prepared by qg_prepare";
    case QG_ERR_WORKSPACE: return "workspace or buffer too small";
    case QG_ERR_CAPACITY: return "MoE align buffers below capacity";
    case QG_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int32_t qg_version(void) { return (1 << 16) | 0; }

size_t qg_prepared_bytes(const qg_layer_desc* desc) {
  if (check_desc(desc, nullptr) != QG_OK) return 0;
  return (size_t)sizes_of(desc).total;
}

qg_status qg_prepare(const qg_layer_desc* desc, const void* w, const void* scales, const void* zeros, void* dev_out,
                     size_t dev_bytes, qg_prepared* out, void* stream) {
  PathInfo pi;
  qg_status s = check_desc(desc, &pi);
  if (s != QG_OK) return s;
  if (!w || !scales || !dev_out || !out) return QG_ERR_INVALID_ARG;
  if (desc->has_zero && !zeros) return QG_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(dev_out) || ((uintptr_t)scales % scale_bytes(desc->s_type)) != 0)
    return QG_ERR_INVALID_ARG;
  const Sizes sz = sizes_of(desc);
  if ((int64_t)dev_bytes < sz.total) return QG_ERR_WORKSPACE;
  s = check_arch();
  if (s != QG_OK) return s;
  RepackArgs a{};
  a.w = w; a.s = scales; a.z = (const uint8_t*)zeros;
  a.out_w = (uint8_t*)dev_out;
  a.out_s = (uint8_t*)dev_out + sz.off_s;
  a.out_z = desc->has_zero ? (uint32_t*)((uint8_t*)dev_out + sz.off_z) : nullptr;
  if (!desc->has_zero) a.z = nullptr;
  a.experts = desc->num_experts; a.n = (int)desc->n; a.k = (int)desc->k; a.groups = (int)sz.groups;
  a.w4 = pi.w4; a.order = pi.order; a.bias8 = pi.bias8; a.s_bytes = scale_bytes(desc->s_type);
  a.s_plain = pi.wp_small == WP_FP8_BLOCK ? sz.sb / 4 * desc->num_experts : 0;
  launch_repack(a, (hipStream_t)stream);
  s = launched();
  if (s != QG_OK) return s;
  qg_prepared p{};
  p.magic = QG_PREPARED_MAGIC; p.layout_version = QG_LAYOUT_VERSION; p.gfx_arch = 950;
  p.desc = *desc; p.dev = dev_out; p.bytes = (uint64_t)sz.total;
  p.off_w = 0; p.off_s = (uint64_t)sz.off_s; p.off_z = (uint64_t)sz.off_z;
  p.w_expert_bytes = (uint64_t)sz.wb; p.s_expert_bytes = (uint64_t)sz.sb; p.z_expert_bytes = (uint64_t)sz.zb;
  *out = p;
  QG_LOG("prepare n=%lld k=%lld experts=%d bytes=%lld", (long long)desc->n, (long long)desc->k,
         desc->num_experts, (long long)sz.total);
  return QG_OK;
}

size_t qg_workspace_bytes(const qg_prepared* p, int64_t m_or_tokens, int32_t topk) {
  PathInfo pi;
  if (check_prepared(p, &pi) != QG_OK || m_or_tokens <= 0) return 0;
  if (topk == 0 && p->desc.num_experts == 1) return dense_workspace(p, pi, m_or_tokens);
  return 0;                                         // grouped products need none
}

static void fill_stream_args(StreamArgs& a, const qg_prepared* p) {
  const uint8_t* base = (const uint8_t*)p->dev;
  a.w = base + p->off_w;
  a.s = base + p->off_s;
  a.z = p->desc.has_zero ? (const uint32_t*)(base + p->off_z) : nullptr;
  a.n = (int)p->desc.n; a.k = (int)p->desc.k; a.group = p->desc.group_k;
  a.w_expert_bytes = (int64_t)p->w_expert_bytes;
  a.s_bytes = (uint32_t)(p->s_expert_bytes * p->desc.num_experts);
  a.z_bytes = (uint32_t)(p->z_expert_bytes * p->desc.num_experts);
}

// W4A4 rows per workgroup of the W4A4 kernel for a dense product: 16 / 32 / 64-row workgroups
// (K split over 8, 8 and 4 waves) while 128 x 128 tiles would leave the GPU under-filled,
// 128 x 128 tiles above; batch-invariant: 128 x 128 tiles for every M (each output then one
// wave's full K loop).  Larger products go to the MFMA kernel before this is asked.
int w4a4_dense_rows(int64_t m, int64_t n, bool binv) {
  if (binv) return 128;
  if (m <= 16) return 16;
  if (m <= 32) return 32;
  const int64_t big = ((m + 127) / 128) * ((n + 127) / 128);
  return big >= 512 ? 128 : 64;
}

// Buffer-resource limits of the kernels: every region a kernel addresses must stay
// below 2^31 bytes (one expert's weights, all scales, the activations).
bool fits_rsrc(const qg_prepared* p, int64_t x_rows) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t row_bytes = p->desc.a_type == QG_A_FP8_E4M3 ? p->desc.k
                            : p->desc.a_type == QG_A_FP4_E2M1 ? p->desc.k / 2 : p->desc.k * 2;
  return (int64_t)p->w_expert_bytes < lim && (int64_t)(p->s_expert_bytes * p->desc.num_experts) < lim &&
         (int64_t)(p->z_expert_bytes * p->desc.num_experts) < lim && x_rows * row_bytes < lim;
}

qg_status qg_gemm(const qg_prepared* p, const void* x, const void* x_scale, void* y, int64_t m, void* ws,
                  size_t ws_bytes, void* stream) {
  PathInfo pi;
  qg_status s = check_prepared(p, &pi);
  if (s != QG_OK) return s;
  if (p->desc.num_experts != 1) return QG_ERR_UNSUPPORTED;
  if (m < 0) return QG_ERR_INVALID_ARG;
  if (m == 0) return QG_OK;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return QG_ERR_INVALID_ARG;
  if ((p->desc.a_type == QG_A_FP8_E4M3 || p->desc.a_type == QG_A_FP4_E2M1) && !x_scale) return QG_ERR_INVALID_ARG;
  if (m > (1 << 24) || !fits_rsrc(p, m)) return QG_ERR_UNSUPPORTED;
  s = check_arch();
  if (s != QG_OK) return s;
  StreamArgs a{};
  fill_stream_args(a, p);
  a.x = x; a.x_scale = (const float*)x_scale; a.y = y; a.m = m; a.x_rows = m;
  a.ksplit = 1;
  if (pi.af == A_FP4) {
    // whole 256-wide K steps and either more than 128 rows or enough 256-column tiles to fill
    // the GPU: the MFMA kernel (activations staged through LDS, 32x32x64 fp4 MFMAs), else the
    // W4A4 kernel.  Above 128 rows the MFMA kernel wins even with fewer tiles than CUs
    // (N = K = 8192, 192..768 rows: 35-40 us against 51-149 us); up to 128 rows the W4A4
    // kernel does (27 against 35-40 us)
    if (!pi.binv && m > 64 && p->desc.k % 256 == 0) {
      MfmaTile t{};
      const int64_t ntiles = (p->desc.n + 255) / 256;
      t.bm = rows256(m, ntiles) ? 256 : 128;   // 256 rows: half the weight feed
      t.grid_x = (unsigned)(((m + t.bm - 1) / t.bm) * ntiles);
      t.grid_y = 1;
      t.ksplit = 1;
      if (t.grid_x >= (unsigned)kCUs || m > 128) {
        QG_LOG("gemm m=%lld n=%lld k=%lld -> fp4 mfma bm=%d grid=%u", (long long)m, (long long)p->desc.n,
               (long long)p->desc.k, t.bm, t.grid_x);
        if (!launch_mfma_gemm(a, t, WP_FP4, A_FP4, pi.of, S_UE8M0, false, false, (hipStream_t)stream))
          return QG_ERR_UNSUPPORTED;
        return launched();
      }
    }
    const int bm = w4a4_dense_rows(m, p->desc.n, pi.binv != 0);
    QG_LOG("gemm m=%lld n=%lld k=%lld -> w4a4 rows=%d", (long long)m, (long long)p->desc.n, (long long)p->desc.k, bm);
    if (!launch_w4a4(a, bm, false, pi.of, 1, (hipStream_t)stream)) return QG_ERR_UNSUPPORTED;
    return launched();
  }
  if (is_block(pi) && (m > dense_stream_max(pi) || pi.binv)) {
    const MfmaTile t = block_tile(m, p->desc.n, p->desc.k, pi);
    if (t.ksplit > 1) {
      const size_t need = dense_workspace(p, pi, m);
      if (!ws || !aligned16(ws) || ws_bytes < need) return QG_ERR_WORKSPACE;
      a.part = (float*)ws;
      a.ksplit = t.ksplit;
    }
    QG_LOG("gemm m=%lld n=%lld k=%lld -> fp8 block-scaled grid=%u ksplit=%d", (long long)m, (long long)p->desc.n,
           (long long)p->desc.k, t.grid_x, t.ksplit);
    if (!launch_mfma_gemm(a, t, pi.wp_mfma, pi.af, pi.of, pi.st, false, false, (hipStream_t)stream))
      return QG_ERR_UNSUPPORTED;
    if (t.ksplit > 1 && !launch_split_reduce(a, false, false, pi.of, (hipStream_t)stream)) return QG_ERR_UNSUPPORTED;
    return launched();
  }
  const bool mfma = m > dense_stream_max(pi) || pi.binv;   // batch-invariant: one MMA type for every M
  if (mfma) {
    const MfmaTile t = mfma_tile(m, p->desc.n, p->desc.k, p->desc.group_k, pi);
    if (t.ksplit > 1) {
      const size_t need = (size_t)t.ksplit * (size_t)m * (size_t)p->desc.n * sizeof(float);
      if (!ws || !aligned16(ws) || ws_bytes < need) return QG_ERR_WORKSPACE;
      a.part = (float*)ws;
      a.ksplit = t.ksplit;
    }
    QG_LOG("gemm m=%lld n=%lld k=%lld -> mfma bm=%d grid=%u ksplit=%d", (long long)m, (long long)p->desc.n,
           (long long)p->desc.k, t.bm, t.grid_x, t.ksplit);
    if (!launch_mfma_gemm(a, t, pi.wp_mfma, pi.af, pi.of, pi.st, p->desc.has_zero != 0, false, (hipStream_t)stream))
      return QG_ERR_UNSUPPORTED;
    if (t.ksplit > 1 &&
        !launch_split_reduce(a, pi.wp_mfma == WP_FP8, pi.af == A_FP8, pi.of, (hipStream_t)stream))
      return QG_ERR_UNSUPPORTED;
    return launched();
  }
  StreamTile t = stream_tile(m, p->desc.n, p->desc.w_type);
  const int sp = stream_split(m, p->desc.n, p->desc.k, p->desc.group_k);
  if (sp > 1) {
    const size_t need = dense_workspace(p, pi, m);
    if (!ws || !aligned16(ws) || ws_bytes < need) return QG_ERR_WORKSPACE;
    t.ncb = 8;
    t.kq = 1;
    t.grid_x = (unsigned)((p->desc.n / 16 + 7) / 8);
    a.part = (float*)ws;
    a.ksplit = sp;
  }
  QG_LOG("gemm m=%lld n=%lld k=%lld -> stream mt=%d grid=%ux%ux%d", (long long)m, (long long)p->desc.n,
         (long long)p->desc.k, t.mt, t.grid_x, t.grid_y, sp);
  if (!launch_stream_gemm(a, t, pi.wp_small, pi.af, pi.of, pi.st, p->desc.has_zero != 0, false, (hipStream_t)stream))
    return QG_ERR_UNSUPPORTED;
  // block-scaled partials are scaled already; the others take their scales in the reduction
  if (sp > 1 && !launch_split_reduce(a, pi.wp_small == WP_FP8, pi.af == A_FP8 && !is_block(pi), pi.of,
                                     (hipStream_t)stream))
    return QG_ERR_UNSUPPORTED;
  return launched();
}

int32_t qg_moe_block_m(const qg_prepared* p, int64_t tokens, int32_t topk) {
  PathInfo pi;
  if (check_prepared(p, &pi) != QG_OK || tokens < 0 || topk <= 0) return 0;
  // With a mean of m rows per expert, counts spread about sqrt(m) (multinomial routing).
  // About one routed row per expert (busy = mean + 3 sqrt(mean) <= 4) streams 4-row blocks; up to a
  // mean of 16 rows, 16-row streaming blocks; above, 128-row MFMA blocks (256 from 512 rows
  // per expert).  Measured against the alternatives at E = 128 top-8 (N = 4096, K = 7168) and
  // E = 64 top-6 (N = 2816, K = 4096): 16-row blocks win up to a mean of 12-16 rows; 32- and
  // 64-row streaming blocks lose to 128-row MFMA blocks (a mean of 36: MXFP4 900 -> 606 us,
  // W4A8 int4 266 -> 135 us, W4A8 MXFP4 562 -> 398 us), except 32-row blocks with 16-bit
  // activations up to a mean of 24 (a mean of 20: 561 against 591 us).  Block-scaled W8A8
  // keeps its streaming blocks up to 64 rows (its streaming kernel wins there, dense too).
  const double rows = (double)tokens * topk;
  const double mean = rows / p->desc.num_experts;
  const double busy = mean + 3.0 * sqrt(mean);
  if (pi.af == A_FP4) {
    // W4A4: 16-row W4A4-kernel blocks while the busier experts fit them, else 128-row blocks
    // (32- and 64-row blocks lost to them: E = 128 top-8, a mean of 8 / 16 / 24 / 36 rows,
    // 446 / 491 / 581 / 650 -> 360 / 366 / 371 / 374 us)
    if (pi.binv) return 128;
    return busy <= 16 ? 16 : 128;
  }
  if (pi.binv) return mean < 512 ? 128 : 256;   // MFMA blocks at every size
  if (busy <= 4) return 4;
  if (is_block(pi) && busy <= 64) return mean <= 16 ? 16 : mean <= 32 ? 32 : 64;
  if (mean <= 16) return 16;
  if (mean <= 24 && pi.af != A_FP8) return 32;
  // 256-row blocks halve the weight conversion per FLOP and add padding rows: int4 weights
  // converted to e4m3 take them from a mean of 128 rows (E = 64 top-6 skewed, K = 4096: a mean
  // of 144 / 192 / 256 / 512 / 768 rows 240 / 319 / 386 / 663 / 943 -> 221 / 293 / 343 / 568 /
  // 802 us; at 72 / 96 rows 128-row blocks win, 149 / 196 against 208 / 215 us), e2m1 weights never (E = 128
  // top-8: a mean of 512 / 768 / 1536 rows 3356 / 4742 / 9102 -> 3020 / 4419 / 8440 us with
  // 128-row blocks under 16-bit activations, 1929 / 2705 -> 1796 / 2534 us under e4m3), the
  // others from a mean of 512.
  const double from256 = pi.wp_mfma == WP_INT4Q_FP8 ? 128 : pi.wp_mfma == WP_FP4 ? 1e300 : 512;
  return mean < from256 ? 128 : 256;
}

qg_status qg_moe_capacity(int64_t tokens, int32_t topk, int32_t num_experts, int32_t block_m, int64_t* cap_sorted,
                          int64_t* cap_blocks) {
  if (tokens < 0 || topk <= 0 || num_experts <= 0 || block_m <= 0 || !cap_sorted || !cap_blocks)
    return QG_ERR_INVALID_ARG;
  const int64_t tk = tokens * topk;
  const int64_t raw = tk + (tk < num_experts ? tk : num_experts) * (int64_t)(block_m - 1);
  *cap_sorted = (raw + block_m - 1) / block_m * block_m;
  *cap_blocks = *cap_sorted / block_m;
  return QG_OK;
}

qg_status qg_moe_align(const int32_t* topk_ids, int64_t tokens, int32_t topk, int32_t num_experts, int32_t block_m,
                       int32_t* sorted_ids, int64_t cap_sorted, int32_t* expert_ids, int64_t cap_blocks,
                       int32_t* num_post_pad, void* stream) {
  if (tokens < 0 || topk <= 0 || num_experts <= 0) return QG_ERR_INVALID_ARG;
  if (block_m <= 0 || block_m > 256 || (block_m & (block_m - 1)) != 0) return QG_ERR_INVALID_ARG;
  if (num_experts > 512) return QG_ERR_UNSUPPORTED;
  if (tokens * topk > (int64_t)1 << 30) return QG_ERR_UNSUPPORTED;
  if (!sorted_ids || !expert_ids || !num_post_pad || (tokens > 0 && !topk_ids)) return QG_ERR_INVALID_ARG;
  int64_t cs, cb;
  qg_moe_capacity(tokens, topk, num_experts, block_m, &cs, &cb);
  if (cap_sorted < cs || cap_blocks < cb) return QG_ERR_CAPACITY;
  qg_status s = check_arch();
  if (s != QG_OK) return s;
  launch_moe_align(topk_ids, (int)(tokens * topk), num_experts, block_m, sorted_ids, cap_sorted, expert_ids,
                   cap_blocks, num_post_pad, (hipStream_t)stream);
  return launched();
}

qg_status qg_moe_grouped_map(int32_t layout, const int32_t* offsets_or_counts, int32_t num_experts, int64_t rows_total,
                             int64_t rows_per_expert, int32_t block_m, int32_t* sorted_ids, int64_t cap_sorted,
                             int32_t* expert_ids, int64_t cap_blocks, int32_t* num_post_pad, void* stream) {
  if (layout != QG_MOE_CONTIGUOUS && layout != QG_MOE_MASKED) return QG_ERR_INVALID_ARG;
  if (num_experts <= 0 || rows_total < 0) return QG_ERR_INVALID_ARG;
  if (block_m <= 0 || block_m > 256 || (block_m & (block_m - 1)) != 0) return QG_ERR_INVALID_ARG;
  if (layout == QG_MOE_MASKED && (rows_per_expert < 0 || rows_total != (int64_t)num_experts * rows_per_expert))
    return QG_ERR_INVALID_ARG;
  if (num_experts > 1024) return QG_ERR_UNSUPPORTED;
  if (rows_total > (int64_t)1 << 30) return QG_ERR_UNSUPPORTED;
  if (!offsets_or_counts || !sorted_ids || !expert_ids || !num_post_pad) return QG_ERR_INVALID_ARG;
  int64_t cs, cb;
  qg_moe_capacity(rows_total, 1, num_experts, block_m, &cs, &cb);
  if (cap_sorted < cs || cap_blocks < cb) return QG_ERR_CAPACITY;
  qg_status s = check_arch();
  if (s != QG_OK) return s;
  if (!launch_grouped_map(offsets_or_counts, layout == QG_MOE_MASKED, num_experts, rows_total, (int)rows_per_expert,
                          block_m, sorted_ids, cs, expert_ids, cb, num_post_pad, (hipStream_t)stream))
    return QG_ERR_UNSUPPORTED;
  return launched();
}

qg_status qg_moe_gemm(const qg_prepared* p, const void* x, const void* x_scale, const int32_t* sorted_ids,
                      const int32_t* expert_ids, const int32_t* num_post_pad, int64_t tokens, int32_t topk,
                      int32_t block_m, void* y, void* ws, size_t ws_bytes, void* stream) {
  PathInfo pi;
  qg_status s = check_prepared(p, &pi);
  if (s != QG_OK) return s;
  if (tokens < 0 || topk <= 0) return QG_ERR_INVALID_ARG;
  if (tokens == 0) return QG_OK;
  if (!x || !y || !sorted_ids || !expert_ids || !num_post_pad || !aligned16(x) || !aligned16(y))
    return QG_ERR_INVALID_ARG;
  if ((p->desc.a_type == QG_A_FP8_E4M3 || p->desc.a_type == QG_A_FP4_E2M1) && !x_scale) return QG_ERR_INVALID_ARG;
  if (block_m != 4 && block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128 && block_m != 256)
    return QG_ERR_UNSUPPORTED;
  if (pi.af == A_FP4 && (block_m == 4 || block_m == 256)) return QG_ERR_UNSUPPORTED;
  if (pi.binv && block_m <= kStreamMaxRows) return QG_ERR_UNSUPPORTED;   // one MMA type for every size
  if (tokens * topk > (int64_t)1 << 30 || !fits_rsrc(p, tokens)) return QG_ERR_UNSUPPORTED;
  s = check_arch();
  if (s != QG_OK) return s;
  int64_t cs, cb;
  qg_moe_capacity(tokens, topk, p->desc.num_experts, block_m, &cs, &cb);
  StreamArgs a{};
  fill_stream_args(a, p);
  a.x = x; a.x_scale = (const float*)x_scale; a.y = y; a.m = 0; a.x_rows = tokens;
  a.sorted_ids = sorted_ids; a.expert_ids = expert_ids; a.num_post_pad = num_post_pad;
  a.topk = topk; a.sentinel = (int)(tokens * topk);
  if (pi.af == A_FP4) {
    if (block_m == 128 && p->desc.k % 256 == 0) {
      MfmaTile t{};
      t.bm = 128;
      t.grid_x = (unsigned)((p->desc.n + 255) / 256);
      t.grid_y = (unsigned)cb;
      t.ksplit = 1;
      QG_LOG("moe_gemm T=%lld topk=%d bm=128 -> fp4 mfma grid=%ux%u", (long long)tokens, topk, t.grid_x, t.grid_y);
      if (!launch_mfma_gemm(a, t, WP_FP4, A_FP4, pi.of, S_UE8M0, false, true, (hipStream_t)stream))
        return QG_ERR_UNSUPPORTED;
      return launched();
    }
    QG_LOG("moe_gemm T=%lld topk=%d bm=%d -> w4a4 grid_y=%lld", (long long)tokens, topk, block_m, (long long)cb);
    if (!launch_w4a4(a, block_m, true, pi.of, (unsigned)cb, (hipStream_t)stream)) return QG_ERR_UNSUPPORTED;
    return launched();
  }
  if (block_m > kStreamMaxRows) {
    MfmaTile t{};
    t.bm = block_m;
    t.grid_x = (unsigned)((p->desc.n + 255) / 256);
    t.grid_y = (unsigned)cb;
    QG_LOG("moe_gemm T=%lld topk=%d bm=%d -> mfma grid=%ux%u", (long long)tokens, topk, block_m, t.grid_x, t.grid_y);
    if (!launch_mfma_gemm(a, t, pi.wp_mfma, pi.af, pi.of, pi.st, p->desc.has_zero != 0, true, (hipStream_t)stream))
      return QG_ERR_UNSUPPORTED;
    return launched();
  }
  StreamTile t = stream_tile(block_m, p->desc.n, p->desc.w_type);
  if (p->desc.w_type != QG_W_FP8_E4M3) {   // 128 columns per workgroup (see launch_mt)
    t.ncb = 8;
    t.kq = 1;
    t.grid_x = (unsigned)((p->desc.n / 16 + 7) / 8);
  }
  t.grid_y = (unsigned)cb;
  QG_LOG("moe_gemm T=%lld topk=%d bm=%d -> stream mt=%d grid=%ux%u", (long long)tokens, topk, block_m, t.mt,
         t.grid_x, t.grid_y);
  if (!launch_stream_gemm(a, t, pi.wp_small, pi.af, pi.of, pi.st, p->desc.has_zero != 0, true, (hipStream_t)stream))
    return QG_ERR_UNSUPPORTED;
  return launched();
}

qg_status qg_moe_swiglu(const void* gate_up, int64_t rows, int64_t inter, int32_t in_type, int32_t out_type, void* out,
                        void* out_scale, void* stream) {
  if (rows < 0 || inter <= 0) return QG_ERR_INVALID_ARG;
  if (in_type != QG_O_F16 && in_type != QG_O_BF16) return QG_ERR_INVALID_ARG;
  if (out_type != QG_A_F16 && out_type != QG_A_BF16 && out_type != QG_A_FP8_E4M3 && out_type != QG_A_FP4_E2M1)
    return QG_ERR_INVALID_ARG;
  if (inter % 8 != 0) return QG_ERR_UNSUPPORTED;
  if (out_type == QG_A_FP8_E4M3 && inter > 8192) return QG_ERR_UNSUPPORTED;
  if (out_type == QG_A_FP4_E2M1 && inter % 32 != 0) return QG_ERR_UNSUPPORTED;
  if (rows > ((int64_t)1 << 31) - 1 || rows * inter > ((int64_t)1 << 40)) return QG_ERR_UNSUPPORTED;
  if (rows == 0) return QG_OK;
  if (!gate_up || !out || !aligned16(gate_up) || !aligned16(out)) return QG_ERR_INVALID_ARG;
  if (out_type == QG_A_FP8_E4M3 && (!out_scale || ((uintptr_t)out_scale & 3u) != 0)) return QG_ERR_INVALID_ARG;
  if (out_type == QG_A_FP4_E2M1 && !out_scale) return QG_ERR_INVALID_ARG;
  qg_status s = check_arch();
  if (s != QG_OK) return s;
  const int in_t = in_type == QG_O_F16 ? O_F16 : O_BF16;
  const int out_t = out_type == QG_A_FP8_E4M3 ? A_FP8
                    : out_type == QG_A_FP4_E2M1 ? A_FP4 : (out_type == QG_A_F16 ? A_F16 : A_BF16);
  const bool scaled = out_type == QG_A_FP8_E4M3 || out_type == QG_A_FP4_E2M1;
  if (!launch_swiglu(gate_up, rows, inter, in_t, out_t, out, scaled ? out_scale : nullptr, (hipStream_t)stream))
    return QG_ERR_UNSUPPORTED;
  return launched();
}

qg_status qg_quantize_e4m3_rows(const void* x, int64_t rows, int64_t k, int32_t in_type, uint8_t* codes, float* scale,
                                void* stream) {
  if (rows < 0 || k <= 0) return QG_ERR_INVALID_ARG;
  if (in_type != QG_A_F16 && in_type != QG_A_BF16) return QG_ERR_INVALID_ARG;
  if (k % 8 != 0 || k > 8192) return QG_ERR_UNSUPPORTED;
  if (rows > ((int64_t)1 << 31) - 1) return QG_ERR_UNSUPPORTED;
  if (rows == 0) return QG_OK;
  if (!x || !codes || !scale || !aligned16(x) || ((uintptr_t)codes & 7u) != 0 || ((uintptr_t)scale & 3u) != 0)
    return QG_ERR_INVALID_ARG;
  qg_status s = check_arch();
  if (s != QG_OK) return s;
  if (!launch_quant_rows_e4m3(x, rows, k, in_type == QG_A_F16 ? O_F16 : O_BF16, codes, scale, (hipStream_t)stream))
    return QG_ERR_UNSUPPORTED;
  return launched();
}

qg_status qg_quantize_e2m1_rows(const void* x, int64_t rows, int64_t k, int32_t in_type, uint8_t* codes,
                                uint8_t* scales, void* stream) {
  if (rows < 0 || k <= 0) return QG_ERR_INVALID_ARG;
  if (in_type != QG_A_F16 && in_type != QG_A_BF16) return QG_ERR_INVALID_ARG;
  if (k % 32 != 0) return QG_ERR_UNSUPPORTED;
  if (rows > ((int64_t)1 << 31) - 1 || rows * (k / 32) > ((int64_t)1 << 36)) return QG_ERR_UNSUPPORTED;
  if (rows == 0) return QG_OK;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return QG_ERR_INVALID_ARG;
  qg_status s = check_arch();
  if (s != QG_OK) return s;
  if (!launch_quant_rows_e2m1(x, rows, k, in_type == QG_A_F16 ? A_F16 : A_BF16, codes, scales, (hipStream_t)stream))
    return QG_ERR_UNSUPPORTED;
  return launched();
}

qg_status qg_moe_combine(const void* y, const float* weights, const int32_t* topk_ids, int64_t tokens, int32_t topk,
                         int32_t num_experts, int64_t n, int32_t dtype, void* out, void* stream) {
  if (tokens < 0 || topk <= 0 || num_experts <= 0 || n <= 0) return QG_ERR_INVALID_ARG;
  if (dtype != QG_O_F16 && dtype != QG_O_BF16) return QG_ERR_INVALID_ARG;
  if (n % 8 != 0) return QG_ERR_UNSUPPORTED;
  if (tokens * topk > ((int64_t)1 << 30) || tokens * n > ((int64_t)1 << 40)) return QG_ERR_UNSUPPORTED;
  if (tokens == 0) return QG_OK;
  if (!y || !weights || !topk_ids || !out || !aligned16(y) || !aligned16(out) || ((uintptr_t)weights & 3u) != 0 ||
      ((uintptr_t)topk_ids & 3u) != 0)
    return QG_ERR_INVALID_ARG;
  qg_status s = check_arch();
  if (s != QG_OK) return s;
  if (!launch_combine(y, weights, topk_ids, tokens, topk, num_experts, n, dtype == QG_O_F16 ? O_F16 : O_BF16, out,
                      (hipStream_t)stream))
    return QG_ERR_UNSUPPORTED;
  return launched();
}

qg_status qg_dequant(const qg_prepared* p, int32_t expert, float* out, void* stream) {
  PathInfo pi;
  qg_status s = check_prepared(p, &pi);
  if (s != QG_OK) return s;
  if (is_block(pi)) return QG_ERR_UNSUPPORTED;   // block scales: the layout check is the byte image
  if (expert < 0 || expert >= p->desc.num_experts || !out) return QG_ERR_INVALID_ARG;
  s = check_arch();
  if (s != QG_OK) return s;
  const uint8_t* base = (const uint8_t*)p->dev;
  DequantArgs a{};
  a.w = base + p->off_w + (int64_t)expert * p->w_expert_bytes;
  a.s = base + p->off_s + (int64_t)expert * p->s_expert_bytes;
  a.z = p->desc.has_zero ? (const uint32_t*)(base + p->off_z + (int64_t)expert * p->z_expert_bytes) : nullptr;
  a.out = out;
  a.n = (int)p->desc.n; a.k = (int)p->desc.k;
  a.groups = p->desc.group_k == 0 ? 1 : (int)(p->desc.k / p->desc.group_k);
  a.group = p->desc.group_k;
  a.wp = pi.dq_wp;   // e2m1 under fp8 / fp4 activations reads back through bf16
  a.af = pi.dq_wp == WP_FP4 && (pi.af == A_FP8 || pi.af == A_FP4) ? A_BF16 : pi.af;
  a.stype = pi.st; a.zero = p->desc.has_zero;
  launch_dequant(a, (hipStream_t)stream);
  return launched();
}

}  // extern "C"

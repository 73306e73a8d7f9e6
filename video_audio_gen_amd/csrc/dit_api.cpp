// The C ABI of the DiT block forward: configuration checks, the weight
// contract and its staging into a caller-owned HBM slab, the batch tables, the
// workspace plan and the launch sequences of the block, the forward and the
// denoise loop.  No device memory is allocated here; no call synchronises the
// host except the staging calls, which copy synchronously by contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <cmath>
#include <vector>

#include "dit.h"
#include "internal.h"
#include "kernels.h"

namespace dit {

static thread_local std::string g_error;

int set_error(int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

static std::atomic<int64_t> g_counters[kCntNum];
void count_launch(Counter c) { g_counters[c].fetch_add(1, std::memory_order_relaxed); }

// Per-launch event timing, off unless dit_profile_begin() was called.
struct ProfRecord {
  int family;
  int ev0, ev1;
};
static std::mutex g_prof_mu;
static std::atomic<bool> g_prof_on{false};
static std::vector<hipEvent_t> g_events;  // pool, reused across passes
static size_t g_events_used = 0;
static std::vector<ProfRecord> g_prof;

static int prof_event() {
  if (g_events_used == g_events.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    g_events.push_back(e);
  }
  return static_cast<int>(g_events_used++);
}

LaunchScope::LaunchScope(Counter c, hipStream_t s) : slot_(-1), s_(s) {
  count_launch(c);
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int a = prof_event(), b = prof_event();
  if (a < 0 || b < 0) return;
  if (hipEventRecord(g_events[a], s) != hipSuccess) return;
  g_prof.push_back({static_cast<int>(c), a, b});
  slot_ = static_cast<int>(g_prof.size()) - 1;
}

LaunchScope::~LaunchScope() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  // a failed record leaves the end event unrecorded: dit_profile_end reports it
  (void)hipEventRecord(g_events[g_prof[slot_].ev1], s_);
}

static bool sync_check_enabled() {
  static const bool on = [] {
    const char* e = getenv("DIT_SYNC_CHECK");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

}  // namespace dit

using namespace dit;

#define DIT_HIP(expr)                                                                       \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return set_error(DIT_E_HIP, "%s: %s (%s)", __func__, hipGetErrorString(e_), #expr);  \
    if (sync_check_enabled()) {                                                             \
      e_ = hipDeviceSynchronize();                                                          \
      if (e_ != hipSuccess)                                                                 \
        return set_error(DIT_E_HIP, "%s: %s after %s", __func__, hipGetErrorString(e_), #expr); \
    }                                                                                       \
  } while (0)

#define DIT_TRY(expr)            \
  do {                           \
    int r_ = (expr);             \
    if (r_ != DIT_OK) return r_; \
  } while (0)

// ============================================================================ config

static int check_config(const dit_config* c) {
  if (c == nullptr) return set_error(DIT_E_INVALID, "config is null");
  if (c->n_blocks < 0 || c->hidden <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->ffn <= 0)
    return set_error(DIT_E_INVALID, "config: non-positive dimension");
  if (c->hidden != c->n_heads * c->head_dim)
    return set_error(DIT_E_INVALID, "config: hidden (%d) != n_heads*head_dim (%d)", c->hidden,
                     c->n_heads * c->head_dim);
  if (c->norm != DIT_NORM_RMS && c->norm != DIT_NORM_LAYER) return set_error(DIT_E_INVALID, "config: norm");
  if (!(c->norm_eps > 0.f)) return set_error(DIT_E_INVALID, "config: norm_eps must be > 0");
  if (c->mlp != DIT_MLP_GATE_UP && c->mlp != DIT_MLP_VALUE_GATE) return set_error(DIT_E_INVALID, "config: mlp");
  if (c->stream_dtype != DIT_F32 && c->stream_dtype != DIT_BF16)
    return set_error(DIT_E_INVALID, "config: stream_dtype");
  if (c->rot_dim <= 0 || c->rot_dim > c->head_dim || c->rot_dim % 2)
    return set_error(DIT_E_INVALID, "config: rot_dim must be even and in (0, head_dim]");
  if (!(c->theta > 0.0)) return set_error(DIT_E_INVALID, "config: theta");
  if (c->cond_dim <= 0) return set_error(DIT_E_INVALID, "config: cond_dim");
  if (c->n_mod < 1 || c->n_mod > DIT_MAX_MODALITIES) return set_error(DIT_E_INVALID, "config: n_mod");
  if (c->io != 0 && c->io != 1) return set_error(DIT_E_INVALID, "config: io must be 0 or 1");
  for (int m = 0; m < c->n_mod; ++m) {
    const dit_modality& md = c->mod[m];
    if (md.n_axes != 1 && md.n_axes != 3) return set_error(DIT_E_INVALID, "config: modality %d n_axes", m);
    int sum = 0;
    for (int a = 0; a < md.n_axes; ++a) {
      if (md.axis_dim[a] <= 0 || md.axis_dim[a] % 2)
        return set_error(DIT_E_INVALID, "config: modality %d axis_dim[%d] must be positive and even", m, a);
      sum += md.axis_dim[a];
    }
    if (sum != c->rot_dim) return set_error(DIT_E_INVALID, "config: modality %d axis dims sum to %d, rot_dim %d", m, sum, c->rot_dim);
    if (c->io) {
      if (md.io != DIT_IO_PATCH3D && md.io != DIT_IO_CHANNEL_MAJOR)
        return set_error(DIT_E_INVALID, "config: modality %d needs an io kind", m);
      if (md.channels <= 0) return set_error(DIT_E_INVALID, "config: modality %d channels", m);
      if (md.io == DIT_IO_PATCH3D) {
        if (md.n_axes != 3) return set_error(DIT_E_INVALID, "config: patch3d modality %d needs 3 axes", m);
        for (int a = 0; a < 3; ++a)
          if (md.patch[a] <= 0) return set_error(DIT_E_INVALID, "config: modality %d patch", m);
      } else if (md.n_axes != 1) {
        return set_error(DIT_E_INVALID, "config: channel-major modality %d needs 1 axis", m);
      }
    } else if (md.io != DIT_IO_NONE) {
      return set_error(DIT_E_INVALID, "config: modality %d has io but config.io == 0", m);
    }
  }
  const bool bf = c->stream_dtype == DIT_BF16;
  if (!modnorm_supported(c->hidden)) return set_error(DIT_E_UNSUPPORTED, "hidden %d: need a multiple of 4, <= 8192", c->hidden);
  if (!rope_split_supported(bf, c->head_dim, c->rot_dim))
    return set_error(DIT_E_UNSUPPORTED, "head_dim %d / rot_dim %d not supported by the rope kernel", c->head_dim, c->rot_dim);
  if (!attention_supported(bf, c->head_dim))
    return set_error(DIT_E_UNSUPPORTED, "head_dim %d not supported by the %s attention kernel", c->head_dim, bf ? "bf16" : "f32");
  if (bf) {
    if (c->hidden % 64 || c->ffn % 64) return set_error(DIT_E_UNSUPPORTED, "bf16 stream needs hidden and ffn multiples of 64");
  } else if (!fused_f32_supported(c->hidden, c->ffn)) {
    return set_error(DIT_E_UNSUPPORTED, "fp32 stream needs ffn a multiple of 4 and <= 24576");
  }
  if (c->cond_dim % 4) return set_error(DIT_E_UNSUPPORTED, "cond_dim must be a multiple of 4");
  if (c->qkv_layout != DIT_QKV_CONCAT && c->qkv_layout != DIT_QKV_PER_HEAD)
    return set_error(DIT_E_INVALID, "config: qkv_layout %d", c->qkv_layout);
  if (c->qk_norm != 0 && c->qk_norm != 1) return set_error(DIT_E_INVALID, "config: qk_norm %d", c->qk_norm);
  if (c->qk_norm && bf) return set_error(DIT_E_UNSUPPORTED, "the q/k norm runs in the fp32 stream only");
  if (c->qk_norm && c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return set_error(DIT_E_UNSUPPORTED, "the q/k norm needs head_dim 32, 64 or 128");
  for (int m = 0; m < c->n_mod; ++m)
    if (c->mod[m].rope_grid != DIT_ROPE_INTEGER && c->mod[m].rope_grid != DIT_ROPE_CENTERED)
      return set_error(DIT_E_INVALID, "config: modality %d rope_grid %d", m, c->mod[m].rope_grid);
  if (c->gemm_format != DIT_GEMM_STREAM && c->gemm_format != DIT_GEMM_MXFP8 && c->gemm_format != DIT_GEMM_MXFP4)
    return set_error(DIT_E_INVALID, "config: gemm_format %d", c->gemm_format);
  if (c->gemm_format != DIT_GEMM_STREAM && (!bf || c->hidden % 128 || c->ffn % 128))
    return set_error(DIT_E_UNSUPPORTED, "MX GEMMs need a bf16 stream and hidden, ffn multiples of 128");
  return DIT_OK;
}

static int token_width(const dit_modality& m) {
  if (m.io == DIT_IO_PATCH3D) return m.channels * m.patch[0] * m.patch[1] * m.patch[2];
  if (m.io == DIT_IO_CHANNEL_MAJOR) return m.channels;
  return 0;
}

// ============================================================================ model and weight contract

enum SlotKind { kBlockMat = 0, kBias = 1, kIsland = 2 };
// Slot dtype of an fp32 GEMM weight: stored as its int8 slices (gemm_f32).
constexpr int kSlicedF32 = 16;
// Slot dtype of an MXFP8 GEMM weight [R, K]: E4M3 codes [R, K], then (256-byte
// aligned) E8M0 scales [R, K/32].
constexpr int kMx8 = 17;
static size_t mx8_bytes(int64_t R, int64_t K) { return ((static_cast<size_t>(R * K) + 255) & ~size_t(255)) + R * K / 32; }
static const uint8_t* mx8_scales(const void* w, int64_t R, int64_t K) {
  return static_cast<const uint8_t*>(w) + ((static_cast<size_t>(R * K) + 255) & ~size_t(255));
}
// Slot dtype of an MXFP4 GEMM weight [R, K]: E2M1 codes [R, K/2], then
// (256-byte aligned) E8M0 scales [R, K/32].
constexpr int kMx4 = 18;
static size_t mx4_bytes(int64_t R, int64_t K) { return ((static_cast<size_t>(R * K / 2) + 255) & ~size_t(255)) + R * K / 32; }
static const uint8_t* mx4_scales(const void* w, int64_t R, int64_t K) {
  return static_cast<const uint8_t*>(w) + ((static_cast<size_t>(R * K / 2) + 255) & ~size_t(255));
}

struct Slot {
  std::string name;
  int ndim;
  int64_t shape[2];
  int dtype;       // slot dtype in the slab
  int kind;
  int row_order;   // kRowsSwapHalves | kRowsPairs32, applied at stage time
  size_t offset, bytes;
  bool staged;
};

struct BlockPtrs {
  const void* adaln_w[DIT_MAX_MODALITIES];
  const float* adaln_b[DIT_MAX_MODALITIES];
  const void *qkv_w, *out_w, *in_w, *mo_w;
  const float *qkv_b, *out_b, *in_b, *mo_b;
  const uint8_t *qkv_s, *out_s, *in_s, *mo_s;  // MXFP8 / MXFP4 weights: their E8M0 scales (else null)
};

struct dit_model {
  dit_config cfg;
  char* slab;
  size_t slab_bytes;
  std::vector<Slot> slots;
  std::unordered_map<std::string, int> index;
  bool finalized;
  dit_stage_stats_t stats;
  std::vector<BlockPtrs> blocks;
  const void* in_w[DIT_MAX_MODALITIES];   // int8 slices
  const float* in_b[DIT_MAX_MODALITIES];
  const void* out_w[DIT_MAX_MODALITIES];  // int8 slices
  const float* out_b[DIT_MAX_MODALITIES];
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Stage-time row orders of the MLP-in weight and bias (2F rows):
//   kRowsSwapHalves: a [value | gate] model is stored [gate | up];
//   kRowsPairs32 (bf16 stream): groups of 64 rows [32 gate | 32 up] of the same
//     32 features, so the GEMM that produces them can apply the SiLU gate in
//     its epilogue (a wave holds both halves of a group).
//   kRowsPerHead (qkv weight and bias, 3D rows): the source is laid out per
//     head [q | k | v of head 0 | ...] (head_dim rows each), stored [q_all |
//     k_all | v_all].
enum RowOrder { kRowsSwapHalves = 1, kRowsPairs32 = 2, kRowsPerHead = 4 };

static int64_t staged_source_row(int64_t r, int64_t rows, int order, int64_t hd) {
  if (order & kRowsPerHead) {
    const int64_t D = rows / 3, part = r / D, hh = (r % D) / hd, d = r % hd;
    return hh * 3 * hd + part * hd + d;
  }
  int64_t q = r;  // row in [gate | up] order
  if (order & kRowsPairs32) {
    const int64_t g = r / 64, w = r % 64;
    q = (w < 32 ? 0 : rows / 2) + g * 32 + (w % 32);
  }
  return (order & kRowsSwapHalves) ? (q + rows / 2) % rows : q;
}

static void build_contract(const dit_config& c, std::vector<Slot>* slots, size_t* total) {
  const int64_t D = c.hidden, F = c.ffn, dt = c.cond_dim;
  const int sd = c.stream_dtype;
  size_t off = 0;
  auto add = [&](const std::string& name, int ndim, int64_t s0, int64_t s1, int dtype, int kind, int order) {
    Slot s;
    s.name = name;
    s.ndim = ndim;
    s.shape[0] = s0;
    s.shape[1] = s1;
    s.dtype = dtype;
    s.kind = kind;
    s.row_order = order;
    const int64_t n = ndim == 1 ? s0 : s0 * s1;
    s.bytes = dtype == kSlicedF32 ? gemm_f32_slices_bytes(static_cast<int>(s0), static_cast<int>(s1))
              : dtype == kMx8     ? mx8_bytes(s0, s1)
              : dtype == kMx4     ? mx4_bytes(s0, s1)
                                  : static_cast<size_t>(n) * (dtype == DIT_BF16 ? 2 : 4);
    s.offset = off;
    s.staged = false;
    off = align256(off + s.bytes);
    slots->push_back(s);
  };
  if (c.io) {
    for (int m = 0; m < c.n_mod; ++m) {
      const int64_t cw = token_width(c.mod[m]);
      add("in." + std::to_string(m) + ".weight", 2, D, cw, kSlicedF32, kIsland, false);
      add("in." + std::to_string(m) + ".bias", 1, D, 0, DIT_F32, kBias, false);
      add("out." + std::to_string(m) + ".weight", 2, cw, D, kSlicedF32, kIsland, false);
      add("out." + std::to_string(m) + ".bias", 1, cw, 0, DIT_F32, kBias, false);
    }
  }
  const int in_order = (c.mlp == DIT_MLP_VALUE_GATE ? kRowsSwapHalves : 0) | (sd == DIT_BF16 ? kRowsPairs32 : 0);
  // dtype of the GEMM weights
  const int gd = sd == DIT_BF16 ? (c.gemm_format == DIT_GEMM_MXFP8 ? kMx8 : c.gemm_format == DIT_GEMM_MXFP4 ? kMx4 : DIT_BF16)
                                 : kSlicedF32;
  for (int b = 0; b < c.n_blocks; ++b) {
    const std::string p = "blocks." + std::to_string(b) + ".";
    for (int m = 0; m < c.n_mod; ++m) {
      add(p + "adaln." + std::to_string(m) + ".weight", 2, 6 * D, dt, sd, kBlockMat, false);
      add(p + "adaln." + std::to_string(m) + ".bias", 1, 6 * D, 0, DIT_F32, kBias, false);
    }
    const int qkv_order = c.qkv_layout == DIT_QKV_PER_HEAD ? kRowsPerHead : 0;
    add(p + "attn.qkv.weight", 2, 3 * D, D, gd, kBlockMat, qkv_order);
    add(p + "attn.qkv.bias", 1, 3 * D, 0, DIT_F32, kBias, qkv_order);
    add(p + "attn.out.weight", 2, D, D, gd, kBlockMat, false);
    add(p + "attn.out.bias", 1, D, 0, DIT_F32, kBias, false);
    add(p + "mlp.in.weight", 2, 2 * F, D, gd, kBlockMat, in_order);
    add(p + "mlp.in.bias", 1, 2 * F, 0, DIT_F32, kBias, in_order);
    add(p + "mlp.out.weight", 2, D, F, gd, kBlockMat, false);
    add(p + "mlp.out.bias", 1, D, 0, DIT_F32, kBias, false);
  }
  *total = off;
}

extern "C" int dit_weight_bytes(const dit_config* cfg, size_t* bytes) {
  DIT_TRY(check_config(cfg));
  if (bytes == nullptr) return set_error(DIT_E_INVALID, "dit_weight_bytes: bytes is null");
  std::vector<Slot> slots;
  build_contract(*cfg, &slots, bytes);
  return DIT_OK;
}

extern "C" int dit_model_create(const dit_config* cfg, void* slab, size_t slab_bytes, dit_model** out) {
  DIT_TRY(check_config(cfg));
  if (out == nullptr) return set_error(DIT_E_INVALID, "dit_model_create: out is null");
  std::vector<Slot> slots;
  size_t need;
  build_contract(*cfg, &slots, &need);
  if (need > 0 && slab == nullptr) return set_error(DIT_E_INVALID, "dit_model_create: weight slab is null");
  if (reinterpret_cast<uintptr_t>(slab) % 256) return set_error(DIT_E_INVALID, "dit_model_create: slab must be 256-byte aligned");
  if (slab_bytes < need)
    return set_error(DIT_E_WORKSPACE, "dit_model_create: slab of %zu bytes, %zu needed", slab_bytes, need);
  dit_model* m = new (std::nothrow) dit_model();
  if (m == nullptr) return set_error(DIT_E_INVALID, "dit_model_create: out of host memory");
  m->cfg = *cfg;
  m->slab = static_cast<char*>(slab);
  m->slab_bytes = slab_bytes;
  m->slots = std::move(slots);
  for (size_t i = 0; i < m->slots.size(); ++i) m->index[m->slots[i].name] = static_cast<int>(i);
  m->finalized = false;
  std::memset(&m->stats, 0, sizeof m->stats);
  *out = m;
  return DIT_OK;
}

extern "C" void dit_model_destroy(dit_model* m) { delete m; }

static inline uint16_t host_f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

extern "C" int dit_stage_weights(dit_model* m, const dit_weight_view* views, int n, dit_stream_t stream) {
  if (m == nullptr || (n > 0 && views == nullptr)) return set_error(DIT_E_INVALID, "dit_stage_weights: null argument");
  if (m->finalized) return set_error(DIT_E_STATE, "dit_stage_weights: staging is already finalized");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::vector<uint8_t> conv, sliced_buf;
  for (int i = 0; i < n; ++i) {
    const dit_weight_view& v = views[i];
    if (v.name == nullptr) return set_error(DIT_E_INVALID, "dit_stage_weights: view %d has no name", i);
    auto it = m->index.find(v.name);
    if (it == m->index.end()) return set_error(DIT_E_UNKNOWN_WEIGHT, "unknown weight '%s'", v.name);
    Slot& sl = m->slots[it->second];
    if (sl.staged) return set_error(DIT_E_INVALID, "weight '%s' staged twice", v.name);
    bool shape_ok = v.ndim == sl.ndim;
    for (int d = 0; shape_ok && d < sl.ndim; ++d) shape_ok = v.shape[d] == sl.shape[d];
    if (!shape_ok) {
      return set_error(DIT_E_SHAPE, "weight '%s': shape mismatch (expected [%lld%s%lld])", v.name,
                       static_cast<long long>(sl.shape[0]), sl.ndim == 2 ? ", " : "",
                       sl.ndim == 2 ? static_cast<long long>(sl.shape[1]) : 0LL);
    }
    if (v.dtype != DIT_F32 && v.dtype != DIT_BF16) return set_error(DIT_E_DTYPE, "weight '%s': dtype %d", v.name, v.dtype);
    if (v.host == nullptr) return set_error(DIT_E_INVALID, "weight '%s': host pointer is null", v.name);
    const int64_t count = sl.ndim == 1 ? sl.shape[0] : sl.shape[0] * sl.shape[1];
    const void* src = v.host;
    const bool sliced = sl.dtype == kSlicedF32;
    const bool mx = sl.dtype == kMx8 || sl.dtype == kMx4;
    const bool need_conv = v.dtype != sl.dtype || sl.row_order != 0;
    if (need_conv) {
      // rows gathered (and widened or rounded) into the slot dtype; a sliced
      // slot gathers float32 rows first and slices them below
      conv.resize(sliced || mx ? sizeof(float) * count : sl.bytes);
      const int64_t rows = sl.shape[0];
      const int64_t cols = sl.ndim == 1 ? 1 : sl.shape[1];
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t sr = staged_source_row(r, rows, sl.row_order, m->cfg.head_dim);
        for (int64_t c = 0; c < cols; ++c) {
          const int64_t di = r * cols + c, si = sr * cols + c;
          if (sl.dtype == DIT_BF16) {
            uint16_t b;
            if (v.dtype == DIT_BF16) b = static_cast<const uint16_t*>(v.host)[si];
            else b = host_f32_to_bf16(static_cast<const float*>(v.host)[si]);
            reinterpret_cast<uint16_t*>(conv.data())[di] = b;
          } else {
            float f;
            if (v.dtype == DIT_F32) {
              f = static_cast<const float*>(v.host)[si];
            } else {
              const uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(v.host)[si]) << 16;
              std::memcpy(&f, &u, 4);
            }
            reinterpret_cast<float*>(conv.data())[di] = f;
          }
        }
      }
      src = conv.data();
      if (mx) {
        // an MX weight is re-quantized from the (bf16) values as given
        sliced_buf.resize(sl.bytes);
        uint8_t* codes = reinterpret_cast<uint8_t*>(sliced_buf.data());
        const float* xs = reinterpret_cast<const float*>(conv.data());
        const int64_t bad =
            sl.dtype == kMx8
                ? host_quantize_mx8(sl.shape[0], sl.shape[1], xs, codes, codes + (mx8_scales(codes, sl.shape[0], sl.shape[1]) - codes))
                : host_quantize_mx4(sl.shape[0], sl.shape[1], xs, codes, codes + (mx4_scales(codes, sl.shape[0], sl.shape[1]) - codes));
        if (bad >= 0)
          return set_error(DIT_E_INVALID, "weight '%s': row %lld holds a NaN or an Inf (MX GEMM weights must be finite)",
                           v.name, static_cast<long long>(bad));
        src = sliced_buf.data();
      }
      if (sliced) {
        sliced_buf.resize(sl.bytes);
        const int64_t bad = host_slice_rows(sl.shape[0], sl.shape[1], (sl.shape[1] + 31) / 32 * 32,
                                            reinterpret_cast<const float*>(conv.data()),
                                            reinterpret_cast<int8_t*>(sliced_buf.data()));
        if (bad >= 0)
          return set_error(DIT_E_INVALID, "weight '%s': row %lld holds a NaN or an Inf (fp32 GEMM weights must be finite)",
                           v.name, static_cast<long long>(bad));
        src = sliced_buf.data();
      }
      const int64_t held = static_cast<int64_t>(conv.size() + sliced_buf.size());
      if (held > m->stats.host_peak) m->stats.host_peak = held;
      m->stats.converted++;
    } else {
      m->stats.direct++;
    }
    (void)count;
    hipError_t e = hipMemcpyAsync(m->slab + sl.offset, src, sl.bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return set_error(DIT_E_HIP, "staging '%s': %s", v.name, hipGetErrorString(e));
    sl.staged = true;
    m->stats.tensors++;
    m->stats.bytes += static_cast<int64_t>(sl.bytes);
    if (conv.capacity() > 0) std::vector<uint8_t>().swap(conv);  // one tensor's buffer at a time
    if (sliced_buf.capacity() > 0) std::vector<uint8_t>().swap(sliced_buf);
  }
  return DIT_OK;
}

extern "C" int dit_stage_finalize(dit_model* m) {
  if (m == nullptr) return set_error(DIT_E_INVALID, "dit_stage_finalize: model is null");
  if (m->finalized) return set_error(DIT_E_STATE, "dit_stage_finalize: already finalized");
  for (const Slot& s : m->slots)
    if (!s.staged) return set_error(DIT_E_MISSING_WEIGHT, "missing weight '%s'", s.name.c_str());
  const dit_config& c = m->cfg;
  auto ptr = [&](const std::string& n) -> char* { return m->slab + m->slots[m->index.at(n)].offset; };
  m->blocks.resize(c.n_blocks);
  for (int b = 0; b < c.n_blocks; ++b) {
    const std::string p = "blocks." + std::to_string(b) + ".";
    BlockPtrs& bp = m->blocks[b];
    for (int mm = 0; mm < DIT_MAX_MODALITIES; ++mm) {
      bp.adaln_w[mm] = mm < c.n_mod ? ptr(p + "adaln." + std::to_string(mm) + ".weight") : nullptr;
      bp.adaln_b[mm] = mm < c.n_mod ? reinterpret_cast<const float*>(ptr(p + "adaln." + std::to_string(mm) + ".bias")) : nullptr;
    }
    bp.qkv_w = ptr(p + "attn.qkv.weight");
    bp.qkv_b = reinterpret_cast<const float*>(ptr(p + "attn.qkv.bias"));
    bp.out_w = ptr(p + "attn.out.weight");
    bp.out_b = reinterpret_cast<const float*>(ptr(p + "attn.out.bias"));
    bp.in_w = ptr(p + "mlp.in.weight");
    bp.in_b = reinterpret_cast<const float*>(ptr(p + "mlp.in.bias"));
    bp.mo_w = ptr(p + "mlp.out.weight");
    bp.mo_b = reinterpret_cast<const float*>(ptr(p + "mlp.out.bias"));
    const int64_t D = c.hidden, F = c.ffn;
    auto scales = [&](const void* w, int64_t R, int64_t K) -> const uint8_t* {
      return c.gemm_format == DIT_GEMM_MXFP8 ? mx8_scales(w, R, K)
             : c.gemm_format == DIT_GEMM_MXFP4 ? mx4_scales(w, R, K)
                                               : nullptr;
    };
    bp.qkv_s = scales(bp.qkv_w, 3 * D, D);
    bp.out_s = scales(bp.out_w, D, D);
    bp.in_s = scales(bp.in_w, 2 * F, D);
    bp.mo_s = scales(bp.mo_w, D, F);
  }
  for (int mm = 0; mm < DIT_MAX_MODALITIES; ++mm) {
    const bool has = c.io && mm < c.n_mod;
    m->in_w[mm] = has ? ptr("in." + std::to_string(mm) + ".weight") : nullptr;
    m->in_b[mm] = has ? reinterpret_cast<const float*>(ptr("in." + std::to_string(mm) + ".bias")) : nullptr;
    m->out_w[mm] = has ? ptr("out." + std::to_string(mm) + ".weight") : nullptr;
    m->out_b[mm] = has ? reinterpret_cast<const float*>(ptr("out." + std::to_string(mm) + ".bias")) : nullptr;
  }
  m->finalized = true;
  return DIT_OK;
}

extern "C" int dit_stage_stats(const dit_model* m, dit_stage_stats_t* out) {
  if (m == nullptr || out == nullptr) return set_error(DIT_E_INVALID, "dit_stage_stats: null argument");
  *out = m->stats;
  return DIT_OK;
}

// ============================================================================ batch

struct dit_batch {
  const dit_model* model;
  int N, n_segs, max_seqlen, n_cond;
  std::vector<dit_segment> segs;
  std::vector<int32_t> cu;          // host copy of cu_seqlens
  std::vector<int> cond_mod;        // modality of each modulation row
  std::vector<int64_t> lat_off;     // float offset of each segment's latent
  int64_t latent_floats;
  int max_seg_tokens;
  const int32_t* cu_dev;
  const int32_t* cond_dev;
  const float* cos_dev;
  const float* sin_dev;
};

struct TableLayout {
  size_t cu, cond, cos, sin, total;
};

static TableLayout table_layout(int N, int n_segs, int half) {
  TableLayout t;
  size_t off = 0;
  t.cu = off;
  off = align256(off + sizeof(int32_t) * (n_segs + 1));
  t.cond = off;
  off = align256(off + sizeof(int32_t) * N);
  t.cos = off;
  off = align256(off + sizeof(float) * static_cast<size_t>(N) * half);
  t.sin = off;
  off = align256(off + sizeof(float) * static_cast<size_t>(N) * half);
  t.total = off;
  return t;
}

static int64_t segment_latent_floats(const dit_config& c, const dit_segment& s) {
  const dit_modality& md = c.mod[s.modality];
  if (md.io == DIT_IO_PATCH3D)
    return static_cast<int64_t>(md.channels) * s.grid[0] * md.patch[0] * s.grid[1] * md.patch[1] * s.grid[2] * md.patch[2];
  if (md.io == DIT_IO_CHANNEL_MAJOR) return static_cast<int64_t>(md.channels) * s.grid[0];
  return 0;
}

extern "C" int dit_batch_bytes(const dit_model* m, const dit_segment* segs, int n_segs, size_t* bytes) {
  if (m == nullptr || bytes == nullptr) return set_error(DIT_E_INVALID, "dit_batch_bytes: null argument");
  std::vector<int32_t> cu(static_cast<size_t>(n_segs > 0 ? n_segs : 0) + 1);
  int N;
  DIT_TRY(dit_pack_layout(&m->cfg, segs, n_segs, cu.data(), nullptr, nullptr, &N));
  *bytes = table_layout(N, n_segs, m->cfg.rot_dim / 2).total;
  return DIT_OK;
}

// Every GEMM a forward over this batch launches must fit the kernels' 32-bit
// buffer offsets (the fp32 GEMM addresses 5 bytes of slices per element of an
// operand, the bf16 GEMM one 256-row tile of an operand at a time).
static int check_gemm_shapes(const dit_config& c, int N, int max_seg_tokens) {
  const int D = c.hidden, F = c.ffn;
  const int shapes[4][2] = {{3 * D, D}, {D, D}, {2 * F, D}, {D, F}};
  for (const auto& sh : shapes) {
    const bool ok = c.stream_dtype == DIT_BF16
                        ? (c.gemm_format != DIT_GEMM_STREAM ? gemm_mx8_supported(N, sh[0], sh[1])
                                                            : gemm_bf16_supported(N, sh[0], sh[1]))
                        : gemm_f32_supported(N, sh[0], sh[1]);
    if (!ok)
      return set_error(DIT_E_UNSUPPORTED, "%s GEMM [%d x %d] x [%d x %d]^T of a %d-token batch is beyond the kernel's 32-bit offsets",
                       c.stream_dtype == DIT_BF16 ? "bf16" : "fp32", N, sh[1], sh[0], sh[1], N);
  }
  if (c.io) {
    for (int mm = 0; mm < c.n_mod; ++mm) {
      const int cw = token_width(c.mod[mm]);
      if (!gemm_f32_supported(max_seg_tokens, D, cw) || !gemm_f32_supported(max_seg_tokens, cw, D))
        return set_error(DIT_E_UNSUPPORTED, "a %d-token segment is beyond the fp32 projection GEMM's 32-bit offsets",
                         max_seg_tokens);
    }
  }
  return DIT_OK;
}

extern "C" int dit_batch_create(const dit_model* m, const dit_segment* segs, int n_segs, int n_cond,
                                const int* cond_modality, void* tables_dev, size_t tables_bytes,
                                dit_stream_t stream, dit_batch** out) {
  if (m == nullptr || out == nullptr || tables_dev == nullptr || cond_modality == nullptr)
    return set_error(DIT_E_INVALID, "dit_batch_create: null argument");
  if (n_cond < 1 || n_cond > DIT_MAX_COND) return set_error(DIT_E_INVALID, "dit_batch_create: n_cond=%d", n_cond);
  const dit_config& c = m->cfg;
  for (int i = 0; i < n_cond; ++i)
    if (cond_modality[i] < 0 || cond_modality[i] >= c.n_mod)
      return set_error(DIT_E_INVALID, "dit_batch_create: cond_modality[%d]=%d", i, cond_modality[i]);
  std::vector<int32_t> cu(static_cast<size_t>(n_segs > 0 ? n_segs : 0) + 1);
  int N;
  DIT_TRY(dit_pack_layout(&c, segs, n_segs, cu.data(), nullptr, nullptr, &N));
  for (int i = 0; i < n_segs; ++i) {
    if (segs[i].cond_row >= n_cond)
      return set_error(DIT_E_INVALID, "dit_batch_create: segment %d uses cond_row %d >= n_cond %d", i, segs[i].cond_row, n_cond);
    if (c.mod[segs[i].modality].n_axes == 1 && (segs[i].grid[1] != 1 || segs[i].grid[2] != 1))
      return set_error(DIT_E_INVALID, "dit_batch_create: segment %d is 1-axis but grid[1..2] != 1", i);
  }
  int max_seg = 0;
  for (int i = 0; i < n_segs; ++i) max_seg = cu[i + 1] - cu[i] > max_seg ? cu[i + 1] - cu[i] : max_seg;
  DIT_TRY(check_gemm_shapes(c, N, max_seg));
  const int half = c.rot_dim / 2;
  TableLayout tl = table_layout(N, n_segs, half);
  if (tables_bytes < tl.total)
    return set_error(DIT_E_WORKSPACE, "dit_batch_create: table buffer of %zu bytes, %zu needed", tables_bytes, tl.total);
  std::vector<uint8_t> host(tl.total, 0);
  std::vector<int32_t> cu2(n_segs + 1);
  DIT_TRY(dit_pack_layout(&c, segs, n_segs, cu2.data(), reinterpret_cast<int32_t*>(host.data() + tl.cond), nullptr, &N));
  std::memcpy(host.data() + tl.cu, cu2.data(), sizeof(int32_t) * (n_segs + 1));
  DIT_TRY(dit_rope_cache_build(&c, segs, n_segs, reinterpret_cast<float*>(host.data() + tl.cos),
                               reinterpret_cast<float*>(host.data() + tl.sin)));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(tables_dev, host.data(), tl.total, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return set_error(DIT_E_HIP, "dit_batch_create: %s", hipGetErrorString(e));

  dit_batch* b = new (std::nothrow) dit_batch();
  if (b == nullptr) return set_error(DIT_E_INVALID, "dit_batch_create: out of host memory");
  b->model = m;
  b->N = N;
  b->n_segs = n_segs;
  b->n_cond = n_cond;
  b->segs.assign(segs, segs + n_segs);
  b->cu = cu2;
  b->cond_mod.assign(cond_modality, cond_modality + n_cond);
  b->max_seqlen = 0;
  b->max_seg_tokens = 0;
  b->latent_floats = 0;
  for (int i = 0; i < n_segs; ++i) {
    const int len = cu2[i + 1] - cu2[i];
    if (len > b->max_seqlen) b->max_seqlen = len;
    b->lat_off.push_back(b->latent_floats);
    b->latent_floats += c.io ? segment_latent_floats(c, segs[i]) : 0;
  }
  b->max_seg_tokens = b->max_seqlen;
  char* base = static_cast<char*>(tables_dev);
  b->cu_dev = reinterpret_cast<const int32_t*>(base + tl.cu);
  b->cond_dev = reinterpret_cast<const int32_t*>(base + tl.cond);
  b->cos_dev = reinterpret_cast<const float*>(base + tl.cos);
  b->sin_dev = reinterpret_cast<const float*>(base + tl.sin);
  *out = b;
  return DIT_OK;
}

extern "C" void dit_batch_destroy(dit_batch* b) { delete b; }

extern "C" int dit_batch_info(const dit_batch* b, int* n_tokens, int* n_segs, int* max_seqlen, int64_t* latent_floats) {
  if (b == nullptr) return set_error(DIT_E_INVALID, "dit_batch_info: batch is null");
  if (n_tokens) *n_tokens = b->N;
  if (n_segs) *n_segs = b->n_segs;
  if (max_seqlen) *max_seqlen = b->max_seqlen;
  if (latent_floats) *latent_floats = b->latent_floats;
  return DIT_OK;
}

extern "C" int dit_batch_tables(const dit_batch* b, const int32_t** cu, const int32_t** cond, const float** cos,
                                const float** sin) {
  if (b == nullptr) return set_error(DIT_E_INVALID, "dit_batch_tables: batch is null");
  if (cu) *cu = b->cu_dev;
  if (cond) *cond = b->cond_dev;
  if (cos) *cos = b->cos_dev;
  if (sin) *sin = b->sin_dev;
  return DIT_OK;
}

// ============================================================================ workspace plan

struct WsPlan {
  size_t mod, x, h, big, qkvh, o, a, sl, gemm, tok, vtok, vel, q8, q8s, total;
};

static size_t gemm_ws(const dit_config& c, int M, int N, int K) {
  return c.stream_dtype == DIT_BF16 ? gemm_bf16_ws_bytes(M, N, K) : gemm_f32_ws_bytes(M, N, K);
}

static WsPlan plan_ws(const dit_model* m, const dit_batch* b) {
  const dit_config& c = m->cfg;
  const size_t N = b->N, D = c.hidden, F = c.ffn;
  const size_t es = c.stream_dtype == DIT_BF16 ? 2 : 4;
  WsPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  p.mod = take(sizeof(float) * c.n_blocks * b->n_cond * 6 * D);
  // residual stream: float32 (bf16 stream, with io) or float64 (fp32 stream)
  p.x = take(c.stream_dtype == DIT_BF16 ? (c.io ? sizeof(float) * N * D : 0) : sizeof(double) * N * D);
  const bool bf = c.stream_dtype == DIT_BF16;
  const bool mx = c.gemm_format != DIT_GEMM_STREAM;  // h and o then live in q8 (MXFP8) only
  p.h = take(bf && !mx ? es * N * D : 0);
  p.big = take(bf ? es * N * 3 * D : 0);  // the QKV GEMM's output (MLP-in's is consumed in its epilogue)
  p.qkvh = take(es * N * (3 * D > F ? 3 * D : F));
  p.o = take(mx ? 0 : es * N * D);
  p.a = take(sizeof(float) * N * D);
  const int Ni = static_cast<int>(N);
  const bool f32 = !bf;
  // fp32 stream: the int8 slices of the next GEMM's input (K = D or F)
  p.sl = take(f32 ? gemm_f32_slices_bytes(Ni, static_cast<int>(D > F ? D : F)) : 0);
  size_t g = 0;
  auto upd = [&](size_t v) { g = v > g ? v : g; };
  if (f32) {  // fp64 split-K partials of the block GEMMs
    upd(gemm_f32_part_bytes(Ni, 3 * D, D));
    upd(gemm_f32_part_bytes(Ni, D, D));
    upd(gemm_f32_part_bytes(Ni, 2 * F, D));
    upd(gemm_f32_part_bytes(Ni, D, F));
  } else {
    upd(gemm_ws(c, Ni, 3 * D, D));
    upd(gemm_ws(c, Ni, D, D));
    upd(gemm_ws(c, Ni, 2 * F, D));
    upd(gemm_ws(c, Ni, D, F));
  }
  size_t tok = 0;
  if (c.io) {
    for (int mm = 0; mm < c.n_mod; ++mm) {
      const int cw = token_width(c.mod[mm]);
      upd(gemm_f32_ws_bytes(b->max_seg_tokens, D, cw));
      upd(gemm_f32_ws_bytes(b->max_seg_tokens, cw, D));
      const size_t t = sizeof(float) * b->max_seg_tokens * cw;
      tok = t > tok ? t : tok;
    }
  }
  p.gemm = take(g);
  p.tok = take(tok);
  p.vtok = take(tok);
  p.vel = take(c.io ? sizeof(float) * b->latent_floats : 0);
  // MX GEMMs: the input of the current GEMM in MXFP8 (h, o, h2: K = D; m: K = F)
  p.q8 = take(mx ? N * (D > F ? D : F) : 0);
  p.q8s = take(mx ? N * (D > F ? D : F) / 32 : 0);
  p.total = off;
  return p;
}

extern "C" int dit_workspace_bytes(const dit_model* m, const dit_batch* b, size_t* bytes) {
  if (m == nullptr || b == nullptr || bytes == nullptr) return set_error(DIT_E_INVALID, "dit_workspace_bytes: null argument");
  if (b->model != m) return set_error(DIT_E_INVALID, "dit_workspace_bytes: batch belongs to another model");
  *bytes = plan_ws(m, b).total;
  return DIT_OK;
}

// ============================================================================ forward

static int check_run(const dit_model* m, const dit_batch* b, void* ws, size_t ws_bytes, WsPlan* plan) {
  if (m == nullptr || b == nullptr) return set_error(DIT_E_INVALID, "model or batch is null");
  if (!m->finalized) return set_error(DIT_E_STATE, "weights are not finalized");
  if (b->model != m) return set_error(DIT_E_INVALID, "batch belongs to another model");
  DIT_TRY(check_gemm_shapes(m->cfg, b->N, b->max_seg_tokens));
  *plan = plan_ws(m, b);
  if (ws_bytes < plan->total)
    return set_error(DIT_E_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, plan->total);
  if (plan->total > 0 && ws == nullptr) return set_error(DIT_E_INVALID, "workspace is null");
  return DIT_OK;
}

// bf16 stream: x is the float32 residual.  h_ready: h already holds this
// block's attention norm (the block before closed with it).  next_mod: the
// next block's modulation rows; the MLP's gated residual then runs fused with
// that block's attention norm, else alone.
static int run_block_bf16(dit_model* m, int blk, float* x, const float* mod, const float* next_mod, bool h_ready,
                          const dit_batch* b, char* ws, const WsPlan& p, hipStream_t s) {
  const dit_config& c = m->cfg;
  const BlockPtrs& w = m->blocks[blk];
  const int N = b->N, D = c.hidden, F = c.ffn, H = c.n_heads, hd = c.head_dim;
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + p.h);
  void* big = ws + p.big;
  uint16_t* qkvh = reinterpret_cast<uint16_t*>(ws + p.qkvh);
  uint16_t* o = reinterpret_cast<uint16_t*>(ws + p.o);
  uint16_t* q = qkvh;
  uint16_t* k = qkvh + static_cast<size_t>(N) * D;
  uint16_t* v = qkvh + 2 * static_cast<size_t>(N) * D;
  // MXFP8 model: the inputs of the QKV, O and MLP-in GEMMs (h, o, h2) are
  // written in MXFP8 (E4M3 codes + E8M0 per 32) by the kernels that produce
  // them -- the norms and the attention -- with the values a quantization of
  // their bf16 form gives; m, which the MLP-in GEMM's SiLU epilogue writes in
  // bf16, is quantized by its own kernel (quantizing inside the GEMM epilogue
  // measured slower: its ALU work runs while the matrix cores idle).  All go
  // to q8 / q8s, each consumed by the GEMM after it.  The MXFP4-weight model
  // runs the same sequence with the weights' FP4 codes as the B operand.
  const bool mx = c.gemm_format != DIT_GEMM_STREAM;
  auto gemm_mx = c.gemm_format == DIT_GEMM_MXFP4 ? gemm_mx4 : gemm_mx8;
  uint8_t* q8 = reinterpret_cast<uint8_t*>(ws + p.q8);
  uint8_t* q8s = reinterpret_cast<uint8_t*>(ws + p.q8s);
  // The SiLU gate runs in the MLP-in GEMM's epilogue (the weight is staged in
  // [32 gate | 32 up] row groups), which writes m = silu(g) * u and never u:
  // every value is the one the separate kernel produces from a stored u.
  float* a = reinterpret_cast<float*>(ws + p.a);
  const GemmEpilogue to_bf16{kEpiBf16};
  const GemmEpilogue to_f32{kEpiF32};
  if (mx) {
    const GemmEpilogue silu{kEpiSiluGate};
    // attention sub-layer
    if (!h_ready) DIT_HIP(modnorm_mx8(c.norm, c.norm_eps, N, D, x, mod, 0, b->cond_dev, q8, q8s, s));
    DIT_HIP(gemm_mx(N, 3 * D, D, q8, q8s, static_cast<const uint8_t*>(w.qkv_w), w.qkv_s, w.qkv_b, big, to_bf16, s));
    DIT_HIP(rope_split(true, N, H, hd, c.rot_dim, big, b->cos_dev, b->sin_dev, q, k, v, s));
    DIT_HIP(attention_bf16(N, H, hd, b->n_segs, b->cu_dev, b->max_seqlen, q, k, v, o, s, q8, q8s));
    DIT_HIP(gemm_mx(N, D, D, q8, q8s, static_cast<const uint8_t*>(w.out_w), w.out_s, w.out_b, a, to_f32, s));
    // MLP sub-layer
    DIT_HIP(resid_modnorm_mx8(c.norm, c.norm_eps, N, D, x, a, mod, 0, mod, 1, b->cond_dev, q8, q8s, s));
    DIT_HIP(gemm_mx(N, 2 * F, D, q8, q8s, static_cast<const uint8_t*>(w.in_w), w.in_s, w.in_b, qkvh, silu, s));
    DIT_HIP(quantize_mx8(N, F, qkvh, q8, q8s, s));
    DIT_HIP(gemm_mx(N, D, F, q8, q8s, static_cast<const uint8_t*>(w.mo_w), w.mo_s, w.mo_b, a, to_f32, s));
    if (next_mod != nullptr)
      DIT_HIP(resid_modnorm_mx8(c.norm, c.norm_eps, N, D, x, a, mod, 1, next_mod, 0, b->cond_dev, q8, q8s, s));
    else
      DIT_HIP(gated_residual(N, D, false, x, a, mod, 1, b->cond_dev, s));
    return DIT_OK;
  }
  const GemmEpilogue silu{kEpiSiluGate};
  auto gemm = [&](int n, int kk, const void* A, const void* W, const float* bias, void* C,
                  const GemmEpilogue& ep) -> hipError_t {
    return gemm_bf16(N, n, kk, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W), bias, C, ep, s);
  };
  // attention sub-layer
  if (!h_ready) DIT_HIP(modnorm(true, c.norm, c.norm_eps, N, D, false, x, mod, 0, b->cond_dev, h, s));
  DIT_HIP(gemm(3 * D, D, h, w.qkv_w, w.qkv_b, big, to_bf16));
  DIT_HIP(rope_split(true, N, H, hd, c.rot_dim, big, b->cos_dev, b->sin_dev, q, k, v, s));
  DIT_HIP(attention_bf16(N, H, hd, b->n_segs, b->cu_dev, b->max_seqlen, q, k, v, o, s));
  DIT_HIP(gemm(D, D, o, w.out_w, w.out_b, a, to_f32));
  // MLP sub-layer: the attention's gated residual and the MLP norm in one pass
  DIT_HIP(resid_modnorm(c.norm, c.norm_eps, N, D, x, a, mod, 0, mod, 1, b->cond_dev, h, s));
  DIT_HIP(gemm(2 * F, D, h, w.in_w, w.in_b, qkvh, silu));
  DIT_HIP(gemm(D, F, qkvh, w.mo_w, w.mo_b, a, to_f32));
  if (next_mod != nullptr)
    DIT_HIP(resid_modnorm(c.norm, c.norm_eps, N, D, x, a, mod, 1, next_mod, 0, b->cond_dev, h, s));
  else
    DIT_HIP(gated_residual(N, D, false, x, a, mod, 1, b->cond_dev, s));
  return DIT_OK;
}

// fp32 stream, x the float64 residual.  Each GEMM reads its input as int8
// slices and leaves fp64 split-K partials that the next row kernel sums (one-
// split column groups finished as fp32, the bias added by the GEMM):
//   (slices of the attention norm, made by the previous block or f32_prologue)
//   QKV GEMM -> rope_part -> attention -> slice_rows -> O GEMM ->
//   resid_norm_slice (gate MSA, MLP norm) -> in GEMM -> silu_slice -> out GEMM ->
//   resid_norm_slice (gate MLP, then next_mod's attention norm sliced, or
//   the plain final norm into y, or nothing)
static int f32_prologue(const dit_model* m, double* x, const float* mod, const dit_batch* b, char* ws,
                        const WsPlan& p, hipStream_t s) {
  const dit_config& c = m->cfg;
  DIT_HIP(resid_norm_slice(b->N, c.hidden, F32Splits{0, 0, c.hidden}, nullptr, nullptr, nullptr, 0, mod, 0, c.norm, c.norm_eps, b->cond_dev, x,
                           ws + p.sl, nullptr, s));
  return DIT_OK;
}

static int run_block_f32(dit_model* m, int blk, double* x, const float* mod, const float* next_mod, float* y,
                         const dit_batch* b, char* ws, const WsPlan& p, hipStream_t s) {
  const dit_config& c = m->cfg;
  const BlockPtrs& w = m->blocks[blk];
  const int N = b->N, D = c.hidden, F = c.ffn, H = c.n_heads, hd = c.head_dim;
  void* sl = ws + p.sl;
  double* part = reinterpret_cast<double*>(ws + p.gemm);
  float* q = reinterpret_cast<float*>(ws + p.qkvh);
  float* k = q + static_cast<size_t>(N) * D;
  float* v = k + static_cast<size_t>(N) * D;
  float* o = reinterpret_cast<float*>(ws + p.o);
  DIT_HIP(gemm_f32_sliced(N, 3 * D, D, sl, w.qkv_w, w.qkv_b, part, s));
  DIT_HIP(rope_part(N, H, hd, c.rot_dim, gemm_f32_split_groups(3 * D, D), part, w.qkv_b, b->cos_dev, b->sin_dev, q, k, v,
                    c.qk_norm, c.norm_eps, s));
  DIT_HIP(attention_f32(N, H, hd, b->n_segs, b->cu_dev, b->max_seqlen, q, k, v, o, s));
  DIT_HIP(slice_rows(N, D, o, sl, s));
  DIT_HIP(gemm_f32_sliced(N, D, D, sl, w.out_w, w.out_b, part, s));
  DIT_HIP(resid_norm_slice(N, D, gemm_f32_split_groups(D, D), part, w.out_b, mod, 0, mod, 1, c.norm, c.norm_eps, b->cond_dev, x,
                           sl, nullptr, s));
  DIT_HIP(gemm_f32_sliced(N, 2 * F, D, sl, w.in_w, w.in_b, part, s));
  DIT_HIP(silu_slice(N, F, gemm_f32_split_groups(2 * F, D), part, w.in_b, sl, s));
  DIT_HIP(gemm_f32_sliced(N, D, F, sl, w.mo_w, w.mo_b, part, s));
  DIT_HIP(resid_norm_slice(N, D, gemm_f32_split_groups(D, F), part, w.mo_b, mod, 1, next_mod, 0, c.norm, c.norm_eps,
                           b->cond_dev, x, next_mod != nullptr ? sl : nullptr, y, s));
  return DIT_OK;
}

static int run_modulation(dit_model* m, const dit_batch* b, int block0, int nb, const float* cond, float* mod,
                          hipStream_t s) {
  const dit_config& c = m->cfg;
  std::vector<AdalnBlockPtrs> ptrs(nb);
  for (int i = 0; i < nb; ++i) {
    for (int mm = 0; mm < 4; ++mm) {
      ptrs[i].w[mm] = m->blocks[block0 + i].adaln_w[mm];
      ptrs[i].bias[mm] = m->blocks[block0 + i].adaln_b[mm];
    }
  }
  DIT_HIP(adaln(c.stream_dtype == DIT_BF16, nb, ptrs.data(), b->n_cond, b->cond_mod.data(), 6 * c.hidden, c.cond_dim,
                cond, mod, s));
  return DIT_OK;
}

extern "C" int dit_modulation(dit_model* m, const dit_batch* b, int block0, int n_blocks, const float* cond_dev,
                              float* mod_dev, dit_stream_t stream) {
  if (m == nullptr || b == nullptr || cond_dev == nullptr || mod_dev == nullptr)
    return set_error(DIT_E_INVALID, "dit_modulation: null argument");
  if (!m->finalized) return set_error(DIT_E_STATE, "dit_modulation: weights are not finalized");
  if (block0 < 0 || n_blocks < 0 || block0 + n_blocks > m->cfg.n_blocks)
    return set_error(DIT_E_INVALID, "dit_modulation: blocks [%d, %d) outside the model", block0, block0 + n_blocks);
  return run_modulation(m, b, block0, n_blocks, cond_dev, mod_dev, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int dit_block_forward(dit_model* m, int block, float* x_dev, const float* mod_dev, const dit_batch* b,
                                 void* ws_dev, size_t ws_bytes, dit_stream_t stream) {
  WsPlan p;
  DIT_TRY(check_run(m, b, ws_dev, ws_bytes, &p));
  if (block < 0 || block >= m->cfg.n_blocks) return set_error(DIT_E_INVALID, "dit_block_forward: block %d", block);
  if (x_dev == nullptr || mod_dev == nullptr) return set_error(DIT_E_INVALID, "dit_block_forward: x or mod is null");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(ws_dev);
  if (m->cfg.stream_dtype == DIT_BF16) return run_block_bf16(m, block, x_dev, mod_dev, nullptr, false, b, ws, p, s);
  const int64_t n = static_cast<int64_t>(b->N) * m->cfg.hidden;
  double* x64 = reinterpret_cast<double*>(ws + p.x);
  DIT_HIP(widen_f32(n, x_dev, x64, s));
  DIT_TRY(f32_prologue(m, x64, mod_dev, b, ws, p, s));
  DIT_TRY(run_block_f32(m, block, x64, mod_dev, nullptr, nullptr, b, ws, p, s));
  DIT_HIP(narrow_f64(n, x64, x_dev, s));
  return DIT_OK;
}

static int run_forward(dit_model* m, const dit_batch* b, const float* in, const float* cond, float* out, char* ws,
                       const WsPlan& p, hipStream_t s) {
  const dit_config& c = m->cfg;
  const int N = b->N, D = c.hidden;
  float* mod = reinterpret_cast<float*>(ws + p.mod);
  DIT_TRY(run_modulation(m, b, 0, c.n_blocks, cond, mod, s));
  // The residual stream: float32 for a bf16 stream, float64 for an fp32 one
  // (entered by exact widening, left rounded once).
  const bool x64 = c.stream_dtype != DIT_BF16;
  const int64_t nd = static_cast<int64_t>(N) * D;
  void* x;
  if (c.io) {
    x = ws + p.x;
    float* xin = x64 ? reinterpret_cast<float*>(ws + p.a) : static_cast<float*>(x);  // in-projection output
    float* tok = reinterpret_cast<float*>(ws + p.tok);
    for (int i = 0; i < b->n_segs; ++i) {
      const dit_segment& sg = b->segs[i];
      const dit_modality& md = c.mod[sg.modality];
      const int n = b->cu[i + 1] - b->cu[i];
      const int cw = token_width(md);
      DIT_HIP(patch_in(md.io, md.channels, md.patch, sg.grid, in + b->lat_off[i], tok, s));
      DIT_HIP(gemm_f32(n, D, cw, tok, m->in_w[sg.modality], m->in_b[sg.modality], xin + static_cast<size_t>(b->cu[i]) * D,
                       ws + p.gemm, s));
    }
    if (x64) DIT_HIP(widen_f32(nd, xin, static_cast<double*>(x), s));
  } else if (x64) {
    x = ws + p.x;
    DIT_HIP(widen_f32(nd, in, static_cast<double*>(x), s));
  } else {
    x = out;
    if (in != out) DIT_HIP(hipMemcpyAsync(out, in, sizeof(float) * N * D, hipMemcpyDeviceToDevice, s));
  }
  const size_t mod_stride = static_cast<size_t>(b->n_cond) * 6 * D;
  float* y = reinterpret_cast<float*>(ws + p.a);  // final norm, fp32
  const int L = c.n_blocks;
  if (x64) {
    // the last block's closing kernel also writes the final norm (with io)
    double* xd = static_cast<double*>(x);
    if (L > 0) DIT_TRY(f32_prologue(m, xd, mod, b, ws, p, s));
    for (int blk = 0; blk < L; ++blk)
      DIT_TRY(run_block_f32(m, blk, xd, mod + blk * mod_stride, blk + 1 < L ? mod + (blk + 1) * mod_stride : nullptr,
                            blk + 1 == L && c.io ? y : nullptr, b, ws, p, s));
  } else {
    for (int blk = 0; blk < L; ++blk)
      DIT_TRY(run_block_bf16(m, blk, static_cast<float*>(x), mod + blk * mod_stride,
                             blk + 1 < L ? mod + (blk + 1) * mod_stride : nullptr, blk > 0, b, ws, p, s));
  }
  if (!c.io) {
    if (x64) DIT_HIP(narrow_f64(nd, static_cast<const double*>(x), out, s));
    return DIT_OK;
  }
  if (!x64 || L == 0) DIT_HIP(modnorm(false, c.norm, c.norm_eps, N, D, x64, x, nullptr, 0, nullptr, y, s));
  float* vtok = reinterpret_cast<float*>(ws + p.vtok);
  for (int i = 0; i < b->n_segs; ++i) {
    const dit_segment& sg = b->segs[i];
    const dit_modality& md = c.mod[sg.modality];
    const int n = b->cu[i + 1] - b->cu[i];
    const int cw = token_width(md);
    DIT_HIP(gemm_f32(n, cw, D, y + static_cast<size_t>(b->cu[i]) * D, m->out_w[sg.modality], m->out_b[sg.modality], vtok,
                     ws + p.gemm, s));
    DIT_HIP(patch_out(md.io, md.channels, md.patch, sg.grid, vtok, out + b->lat_off[i], s));
  }
  return DIT_OK;
}

extern "C" int dit_forward(dit_model* m, const dit_batch* b, const float* in_dev, const float* cond_dev, float* out_dev,
                           void* ws_dev, size_t ws_bytes, dit_stream_t stream) {
  WsPlan p;
  DIT_TRY(check_run(m, b, ws_dev, ws_bytes, &p));
  if (in_dev == nullptr || cond_dev == nullptr || out_dev == nullptr)
    return set_error(DIT_E_INVALID, "dit_forward: null input, cond or output");
  return run_forward(m, b, in_dev, cond_dev, out_dev, static_cast<char*>(ws_dev), p,
                     reinterpret_cast<hipStream_t>(stream));
}

static int run_step(dit_model* m, const dit_batch* b, float* lat, const float* cond, const float* dt, char* ws,
                    const WsPlan& p, hipStream_t s) {
  float* vel = reinterpret_cast<float*>(ws + p.vel);
  DIT_TRY(run_forward(m, b, lat, cond, vel, ws, p, s));
  for (int i = 0; i < b->n_segs; ++i) {
    const int64_t n = (i + 1 < b->n_segs ? b->lat_off[i + 1] : b->latent_floats) - b->lat_off[i];
    DIT_HIP(euler(n, lat + b->lat_off[i], vel + b->lat_off[i], dt + b->segs[i].modality, s));
  }
  return DIT_OK;
}

extern "C" int dit_denoise_step(dit_model* m, const dit_batch* b, float* latents_dev, const float* cond_dev,
                                const float* dt_dev, void* ws_dev, size_t ws_bytes, dit_stream_t stream) {
  WsPlan p;
  DIT_TRY(check_run(m, b, ws_dev, ws_bytes, &p));
  if (!m->cfg.io) return set_error(DIT_E_INVALID, "dit_denoise_step: the model has no latent io");
  if (latents_dev == nullptr || cond_dev == nullptr || dt_dev == nullptr)
    return set_error(DIT_E_INVALID, "dit_denoise_step: null argument");
  return run_step(m, b, latents_dev, cond_dev, dt_dev, static_cast<char*>(ws_dev), p,
                  reinterpret_cast<hipStream_t>(stream));
}

extern "C" int dit_denoise_loop(dit_model* m, const dit_batch* b, float* latents_dev, const float* cond_table_dev,
                                const float* dt_table_dev, int n_steps, void* ws_dev, size_t ws_bytes,
                                dit_stream_t stream) {
  WsPlan p;
  DIT_TRY(check_run(m, b, ws_dev, ws_bytes, &p));
  if (!m->cfg.io) return set_error(DIT_E_INVALID, "dit_denoise_loop: the model has no latent io");
  if (latents_dev == nullptr || cond_table_dev == nullptr || dt_table_dev == nullptr || n_steps < 0)
    return set_error(DIT_E_INVALID, "dit_denoise_loop: bad argument");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t cstride = static_cast<size_t>(b->n_cond) * m->cfg.cond_dim;
  for (int i = 0; i < n_steps; ++i)
    DIT_TRY(run_step(m, b, latents_dev, cond_table_dev + i * cstride, dt_table_dev + static_cast<size_t>(i) * m->cfg.n_mod,
                     static_cast<char*>(ws_dev), p, s));
  return DIT_OK;
}

// Guided loop: the batch holds 2P segments, segment j + P the unconditional
// branch of segment j on the same latent.  Each step copies the P latents
// into both halves of the velocity buffer, runs the forward in place there
// (the forward reads its whole input before it writes its output), then moves
// latent j by dt times the guided velocity of pair j.
static int check_cfg_pairs(const dit_batch* b, int* P) {
  if (b->n_segs % 2) return set_error(DIT_E_INVALID, "guided loop: %d segments, an even count is needed", b->n_segs);
  const int h = b->n_segs / 2;
  for (int j = 0; j < h; ++j) {
    const dit_segment& a = b->segs[j];
    const dit_segment& u = b->segs[j + h];
    if (a.modality != u.modality || a.grid[0] != u.grid[0] || a.grid[1] != u.grid[1] || a.grid[2] != u.grid[2])
      return set_error(DIT_E_INVALID, "guided loop: segments %d and %d do not pair (modality or grid differ)", j, j + h);
    if (b->lat_off[j + h] - b->lat_off[h] != b->lat_off[j])
      return set_error(DIT_E_INVALID, "guided loop: latent layout of segment %d does not mirror segment %d", j + h, j);
  }
  *P = h;
  return DIT_OK;
}

extern "C" int dit_cfg_denoise_loop(dit_model* m, const dit_batch* b, float* latents_dev, const float* cond_table_dev,
                                    const float* dt_table_dev, float w, int n_steps, void* ws_dev, size_t ws_bytes,
                                    dit_stream_t stream) {
  WsPlan p;
  DIT_TRY(check_run(m, b, ws_dev, ws_bytes, &p));
  if (!m->cfg.io) return set_error(DIT_E_INVALID, "dit_cfg_denoise_loop: the model has no latent io");
  if (latents_dev == nullptr || cond_table_dev == nullptr || dt_table_dev == nullptr || n_steps < 0)
    return set_error(DIT_E_INVALID, "dit_cfg_denoise_loop: bad argument");
  if (!std::isfinite(w)) return set_error(DIT_E_INVALID, "dit_cfg_denoise_loop: guidance weight is not finite");
  int P = 0;
  DIT_TRY(check_cfg_pairs(b, &P));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(ws_dev);
  float* vel = reinterpret_cast<float*>(ws + p.vel);
  const int64_t half = b->lat_off[P];  // floats of the P shared latents
  const size_t cstride = static_cast<size_t>(b->n_cond) * m->cfg.cond_dim;
  for (int i = 0; i < n_steps; ++i) {
    DIT_HIP(hipMemcpyAsync(vel, latents_dev, sizeof(float) * half, hipMemcpyDeviceToDevice, s));
    DIT_HIP(hipMemcpyAsync(vel + half, latents_dev, sizeof(float) * half, hipMemcpyDeviceToDevice, s));
    DIT_TRY(run_forward(m, b, vel, cond_table_dev + i * cstride, vel, ws, p, s));
    const float* dt = dt_table_dev + static_cast<size_t>(i) * m->cfg.n_mod;
    for (int j = 0; j < P; ++j) {
      const int64_t n = (j + 1 < P ? b->lat_off[j + 1] : half) - b->lat_off[j];
      DIT_HIP(cfg_euler(n, latents_dev + b->lat_off[j], vel + b->lat_off[j], vel + half + b->lat_off[j], w,
                        dt + b->segs[j].modality, s));
    }
  }
  return DIT_OK;
}

// ============================================================================ captured forwards
// One forward's launches recorded once into a HIP graph and replayed as a
// single launch: the kernels, their arguments and the buffers are fixed at
// capture, the buffers' contents are read when the graph runs.
struct dit_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  size_t nodes = 0;
};

extern "C" int dit_forward_graph_create(dit_model* m, const dit_batch* b, const float* in_dev, const float* cond_dev,
                                        float* out_dev, void* ws_dev, size_t ws_bytes, dit_graph** out) {
  if (out == nullptr) return set_error(DIT_E_INVALID, "dit_forward_graph_create: null output handle");
  *out = nullptr;
  WsPlan p;
  DIT_TRY(check_run(m, b, ws_dev, ws_bytes, &p));
  if (in_dev == nullptr || cond_dev == nullptr || out_dev == nullptr)
    return set_error(DIT_E_INVALID, "dit_forward_graph_create: null input, cond or output");
  if (sync_check_enabled())
    return set_error(DIT_E_UNSUPPORTED, "dit_forward_graph_create: DIT_SYNC_CHECK synchronises after every launch, "
                                        "which a capture cannot record");
  if (g_prof_on.load())
    return set_error(DIT_E_UNSUPPORTED, "dit_forward_graph_create: per-launch profiling is on (dit_profile_begin); "
                                        "end it before capturing");
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return set_error(DIT_E_HIP, "dit_forward_graph_create: %s", hipGetErrorString(e));
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return set_error(DIT_E_HIP, "dit_forward_graph_create: begin capture: %s", hipGetErrorString(e));
  }
  const int r = run_forward(m, b, in_dev, cond_dev, out_dev, static_cast<char*>(ws_dev), p, cs);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);  // always ends the capture, also after a failed launch
  (void)hipStreamDestroy(cs);
  if (r != DIT_OK || e != hipSuccess || g == nullptr) {
    if (g != nullptr) (void)hipGraphDestroy(g);
    return r != DIT_OK ? r : set_error(DIT_E_HIP, "dit_forward_graph_create: end capture: %s", hipGetErrorString(e));
  }
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return set_error(DIT_E_HIP, "dit_forward_graph_create: instantiate: %s", hipGetErrorString(e));
  }
  dit_graph* h = new dit_graph;
  h->graph = g;
  h->exec = x;
  (void)hipGraphGetNodes(g, nullptr, &h->nodes);
  *out = h;
  return DIT_OK;
}

extern "C" int dit_graph_launch(dit_graph* g, dit_stream_t stream) {
  if (g == nullptr) return set_error(DIT_E_INVALID, "dit_graph_launch: null graph");
  DIT_HIP(hipGraphLaunch(g->exec, reinterpret_cast<hipStream_t>(stream)));
  return DIT_OK;
}

extern "C" int dit_graph_nodes(const dit_graph* g, size_t* nodes) {
  if (g == nullptr || nodes == nullptr) return set_error(DIT_E_INVALID, "dit_graph_nodes: null argument");
  *nodes = g->nodes;
  return DIT_OK;
}

extern "C" void dit_graph_destroy(dit_graph* g) {
  if (g == nullptr) return;
  if (g->exec != nullptr) (void)hipGraphExecDestroy(g->exec);
  if (g->graph != nullptr) (void)hipGraphDestroy(g->graph);
  delete g;
}

// ============================================================================ op-level calls

extern "C" int dit_gemm_splits(int dtype, int N, int K, int* splits) {
  if (splits == nullptr || dtype != DIT_F32 || N <= 0 || K <= 0) return set_error(DIT_E_INVALID, "dit_gemm_splits: bad argument");
  *splits = gemm_f32_splits(N, K);
  return DIT_OK;
}

extern "C" int dit_gemm_split_groups(int dtype, int N, int K, int* s_lo, int* s_hi, int* col_split) {
  if (s_lo == nullptr || s_hi == nullptr || col_split == nullptr || dtype != DIT_F32 || N <= 0 || K <= 0)
    return set_error(DIT_E_INVALID, "dit_gemm_split_groups: bad argument");
  const F32Splits g = gemm_f32_split_groups(N, K);
  *s_lo = g.s_lo;
  *s_hi = g.s_hi;
  *col_split = g.col_split;
  return DIT_OK;
}

extern "C" int dit_gemm_workspace_bytes(int dtype, int M, int N, int K, size_t* bytes) {
  if (bytes == nullptr || M < 0 || N <= 0 || K <= 0) return set_error(DIT_E_INVALID, "dit_gemm_workspace_bytes: bad argument");
  // f32: the slices of B, then the GEMM's own scratch (slices of A, split-K partials);
  // MXFP8 / MXFP4: both operands re-quantized (codes, then scales)
  *bytes = dtype == DIT_BF16    ? gemm_bf16_ws_bytes(M, N, K)
           : dtype == DIT_MXFP8 ? (K % 32 ? 0 : mx8_bytes(M, K) + 256 + mx8_bytes(N, K))
           : dtype == DIT_MXFP4 ? (K % 32 ? 0 : mx8_bytes(M, K) + 256 + mx4_bytes(N, K))
                                : gemm_f32_slices_bytes(N, K) + gemm_f32_ws_bytes(M, N, K);
  return DIT_OK;
}

extern "C" int dit_gemm(int dtype, int M, int N, int K, const void* A, const void* B, const float* bias, void* C,
                        int c_dtype, void* ws, size_t ws_bytes, dit_stream_t stream) {
  if (M < 0 || N <= 0 || K <= 0) return set_error(DIT_E_INVALID, "dit_gemm: M=%d N=%d K=%d", M, N, K);
  if (M > 0 && (A == nullptr || B == nullptr || C == nullptr)) return set_error(DIT_E_INVALID, "dit_gemm: null operand");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == DIT_BF16) {
    if (!gemm_bf16_supported(M, N, K)) return set_error(DIT_E_UNSUPPORTED, "dit_gemm bf16: K=%d must be a multiple of 64", K);
    if (c_dtype != DIT_F32 && c_dtype != DIT_BF16) return set_error(DIT_E_INVALID, "dit_gemm: c_dtype");
    const GemmEpilogue ep{c_dtype == DIT_F32 ? kEpiF32 : kEpiBf16};
    DIT_HIP(gemm_bf16(M, N, K, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), bias, C, ep, s));
    return DIT_OK;
  }
  if (dtype == DIT_MXFP8 || dtype == DIT_MXFP4) {
    // A [M,K] and B [N,K] bf16, re-quantized into ws (A to MXFP8, B to MXFP8
    // or MXFP4), then the scaled MX GEMM
    const bool four = dtype == DIT_MXFP4;
    const char* nm = four ? "mxfp4" : "mxfp8";
    if (!gemm_mx8_supported(M, N, K)) return set_error(DIT_E_UNSUPPORTED, "dit_gemm %s: K=%d must be a multiple of 128", nm, K);
    if (c_dtype != DIT_F32 && c_dtype != DIT_BF16) return set_error(DIT_E_INVALID, "dit_gemm: c_dtype");
    const size_t need = mx8_bytes(M, K) + 256 + (four ? mx4_bytes(N, K) : mx8_bytes(N, K));
    if (ws_bytes < need) return set_error(DIT_E_WORKSPACE, "dit_gemm: workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (ws == nullptr) return set_error(DIT_E_INVALID, "dit_gemm: workspace is null");
    if (M == 0) return DIT_OK;
    uint8_t* qa = static_cast<uint8_t*>(ws);
    uint8_t* qb = qa + align256(mx8_bytes(M, K));
    const uint8_t* sa = mx8_scales(qa, M, K);
    const uint8_t* sb = four ? mx4_scales(qb, N, K) : mx8_scales(qb, N, K);
    DIT_HIP(quantize_mx8(M, K, static_cast<const uint16_t*>(A), qa, const_cast<uint8_t*>(sa), s));
    if (four)
      DIT_HIP(quantize_mx4(N, K, static_cast<const uint16_t*>(B), qb, const_cast<uint8_t*>(sb), s));
    else
      DIT_HIP(quantize_mx8(N, K, static_cast<const uint16_t*>(B), qb, const_cast<uint8_t*>(sb), s));
    const GemmEpilogue ep{c_dtype == DIT_F32 ? kEpiF32 : kEpiBf16};
    if (four)
      DIT_HIP(gemm_mx4(M, N, K, qa, sa, qb, sb, bias, C, ep, s));
    else
      DIT_HIP(gemm_mx8(M, N, K, qa, sa, qb, sb, bias, C, ep, s));
    return DIT_OK;
  }
  if (dtype != DIT_F32) return set_error(DIT_E_INVALID, "dit_gemm: dtype");
  if (c_dtype != DIT_F32) return set_error(DIT_E_INVALID, "dit_gemm f32: C must be f32");
  if (!gemm_f32_supported(M, N, K))
    return set_error(DIT_E_UNSUPPORTED, "dit_gemm f32: K=%d must be a multiple of 4 (and slices within 2 GB)", K);
  const size_t bsl = gemm_f32_slices_bytes(N, K);
  const size_t need = bsl + gemm_f32_ws_bytes(M, N, K);
  if (ws_bytes < need) return set_error(DIT_E_WORKSPACE, "dit_gemm: workspace of %zu bytes, %zu needed", ws_bytes, need);
  if (ws == nullptr) return set_error(DIT_E_INVALID, "dit_gemm: workspace is null");
  if (M == 0) return DIT_OK;
  DIT_HIP(slice_rows(N, K, static_cast<const float*>(B), ws, s));
  DIT_HIP(gemm_f32(M, N, K, static_cast<const float*>(A), ws, bias, static_cast<float*>(C), static_cast<char*>(ws) + bsl, s));
  return DIT_OK;
}

extern "C" int dit_quantize_mx8(int R, int K, const void* x, void* codes, void* scales, dit_stream_t stream) {
  if (R < 0 || K <= 0 || K % 32) return set_error(DIT_E_INVALID, "dit_quantize_mx8: R=%d K=%d (K a multiple of 32)", R, K);
  if (R > 0 && (x == nullptr || codes == nullptr || scales == nullptr))
    return set_error(DIT_E_INVALID, "dit_quantize_mx8: null pointer");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(codes)) & 15)
    return set_error(DIT_E_INVALID, "dit_quantize_mx8: x and codes must be 16-byte aligned");
  DIT_HIP(quantize_mx8(R, K, static_cast<const uint16_t*>(x), static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                       reinterpret_cast<hipStream_t>(stream)));
  return DIT_OK;
}

extern "C" int dit_quantize_mx4(int R, int K, const void* x, void* codes, void* scales, dit_stream_t stream) {
  if (R < 0 || K <= 0 || K % 32) return set_error(DIT_E_INVALID, "dit_quantize_mx4: R=%d K=%d (K a multiple of 32)", R, K);
  if (R > 0 && (x == nullptr || codes == nullptr || scales == nullptr))
    return set_error(DIT_E_INVALID, "dit_quantize_mx4: null pointer");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(codes)) & 15)
    return set_error(DIT_E_INVALID, "dit_quantize_mx4: x and codes must be 16-byte aligned");
  DIT_HIP(quantize_mx4(R, K, static_cast<const uint16_t*>(x), static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                       reinterpret_cast<hipStream_t>(stream)));
  return DIT_OK;
}

extern "C" int dit_modnorm(int dtype, int norm, float eps, int N, int D, const void* x, int x_dtype, const float* mod,
                           int which, const int32_t* cond_idx, void* h, dit_stream_t stream) {
  if (N < 0 || !modnorm_supported(D)) return set_error(DIT_E_INVALID, "dit_modnorm: N=%d D=%d", N, D);
  if (norm != DIT_NORM_RMS && norm != DIT_NORM_LAYER) return set_error(DIT_E_INVALID, "dit_modnorm: norm");
  if (which != 0 && which != 1) return set_error(DIT_E_INVALID, "dit_modnorm: which");
  if (mod != nullptr && cond_idx == nullptr) return set_error(DIT_E_INVALID, "dit_modnorm: cond_idx is null");
  if (dtype != DIT_F32 && dtype != DIT_BF16) return set_error(DIT_E_INVALID, "dit_modnorm: dtype");
  if (x_dtype != DIT_F32 && !(x_dtype == DIT_F64 && dtype == DIT_F32))
    return set_error(DIT_E_INVALID, "dit_modnorm: x_dtype %d with output dtype %d", x_dtype, dtype);
  DIT_HIP(modnorm(dtype == DIT_BF16, norm, eps, N, D, x_dtype == DIT_F64, x, mod, which, cond_idx, h,
                  reinterpret_cast<hipStream_t>(stream)));
  return DIT_OK;
}

extern "C" int dit_rope_split(int dtype, int N, int H, int hd, int rot, const void* qkv, const float* cos, const float* sin,
                              void* q, void* k, void* v, dit_stream_t stream) {
  const bool bf = dtype == DIT_BF16;
  if (N < 0 || H <= 0 || !rope_split_supported(bf, hd, rot)) return set_error(DIT_E_INVALID, "dit_rope_split: shape");
  DIT_HIP(rope_split(bf, N, H, hd, rot, qkv, cos, sin, q, k, v, reinterpret_cast<hipStream_t>(stream)));
  return DIT_OK;
}

extern "C" int dit_attention(int dtype, int N, int H, int hd, int n_docs, const int32_t* cu, int max_seqlen, const void* q,
                             const void* k, const void* v, void* o, dit_stream_t stream) {
  const bool bf = dtype == DIT_BF16;
  if (N < 0 || H <= 0 || n_docs < 0 || max_seqlen < 0 || !attention_supported(bf, hd))
    return set_error(DIT_E_INVALID, "dit_attention: shape");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (bf)
    DIT_HIP(attention_bf16(N, H, hd, n_docs, cu, max_seqlen, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), s));
  else
    DIT_HIP(attention_f32(N, H, hd, n_docs, cu, max_seqlen, static_cast<const float*>(q), static_cast<const float*>(k),
                          static_cast<const float*>(v), static_cast<float*>(o), s));
  return DIT_OK;
}

extern "C" int dit_silu_gate(int dtype, int N, int F, const void* u, void* m, dit_stream_t stream) {
  const bool bf = dtype == DIT_BF16;
  if (N < 0 || F <= 0 || F % (bf ? 8 : 4)) return set_error(DIT_E_INVALID, "dit_silu_gate: F=%d", F);
  DIT_HIP(silu_gate(bf, N, F, u, m, reinterpret_cast<hipStream_t>(stream)));
  return DIT_OK;
}

extern "C" int dit_gated_residual(int N, int D, void* x, int x_dtype, const float* a, const float* mod, int which,
                                  const int32_t* cond_idx, dit_stream_t stream) {
  if (N < 0 || D <= 0 || D % 4 || (which != 0 && which != 1)) return set_error(DIT_E_INVALID, "dit_gated_residual: shape");
  if (x_dtype != DIT_F32 && x_dtype != DIT_F64) return set_error(DIT_E_INVALID, "dit_gated_residual: x_dtype %d", x_dtype);
  DIT_HIP(gated_residual(N, D, x_dtype == DIT_F64, x, a, mod, which, cond_idx, reinterpret_cast<hipStream_t>(stream)));
  return DIT_OK;
}

// ============================================================================ diagnostics

extern "C" const char* dit_last_error(void) { return g_error.c_str(); }

extern "C" int dit_counters(int64_t* out, int n_max) {
  if (out == nullptr) return set_error(DIT_E_INVALID, "dit_counters: out is null");
  for (int i = 0; i < n_max && i < kCntNum; ++i) out[i] = g_counters[i].load();
  return DIT_OK;
}

extern "C" void dit_counters_reset(void) {
  for (int i = 0; i < kCntNum; ++i) g_counters[i].store(0);
}

extern "C" int dit_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.clear();
  g_events_used = 0;
  g_prof_on.store(true);
  return DIT_OK;
}

extern "C" int dit_profile_end(int64_t* counts, double* total_ms, int n_max) {
  g_prof_on.store(false);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (counts == nullptr || total_ms == nullptr) return set_error(DIT_E_INVALID, "dit_profile_end: null output");
  for (int i = 0; i < n_max; ++i) {
    counts[i] = 0;
    total_ms[i] = 0.0;
  }
  for (const ProfRecord& r : g_prof) {
    hipError_t e = hipEventSynchronize(g_events[r.ev1]);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_events[r.ev0], g_events[r.ev1]);
    if (e != hipSuccess) return set_error(DIT_E_HIP, "dit_profile_end: %s", hipGetErrorString(e));
    if (r.family < n_max) {
      counts[r.family] += 1;
      total_ms[r.family] += ms;
    }
  }
  g_prof.clear();
  g_events_used = 0;
  return DIT_OK;
}

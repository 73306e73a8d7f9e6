// Host-side tables built in fp64 before any kernel runs: packed layout, per-row
// RoPE cos/sin cache, sinusoidal timestep embedding and the sigma schedule.
// Compiled with -ffp-contract=off so every product and sum rounds on its own,
// which makes the tables reproducible bit for bit from their definitions.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "dit.h"
#include "internal.h"

using dit::set_error;

static int segment_tokens(const dit_config* cfg, const dit_segment& s, int64_t* n) {
  if (s.modality < 0 || s.modality >= cfg->n_mod) return -1;
  const int axes = cfg->mod[s.modality].n_axes;
  int64_t t = 1;
  for (int a = 0; a < axes; ++a) {
    if (s.grid[a] <= 0) return -1;
    t *= s.grid[a];
  }
  *n = t;
  return 0;
}

// Page "port the MiniMax-H3 omni-modal video+audio DiT", section "Correctness
// gates": packed layout (ids, tags, cu_seqlens, doc ids) gated exact.
extern "C" int dit_pack_layout(const dit_config* cfg, const dit_segment* segs, int n_segs,
                               int32_t* cu_seqlens, int32_t* cond_idx, int32_t* doc_id,
                               int* n_tokens) {
  if (cfg == nullptr || segs == nullptr || cu_seqlens == nullptr || n_tokens == nullptr)
    return set_error(DIT_E_INVALID, "dit_pack_layout: null argument");
  if (n_segs < 1 || n_segs > DIT_MAX_SEGMENTS)
    return set_error(DIT_E_INVALID, "dit_pack_layout: n_segs=%d outside [1, %d]", n_segs,
                     DIT_MAX_SEGMENTS);
  int64_t total = 0;
  cu_seqlens[0] = 0;
  for (int i = 0; i < n_segs; ++i) {
    int64_t n;
    if (segment_tokens(cfg, segs[i], &n) != 0)
      return set_error(DIT_E_INVALID, "dit_pack_layout: segment %d has a bad modality or extent", i);
    if (segs[i].cond_row < 0 || segs[i].cond_row >= DIT_MAX_COND)
      return set_error(DIT_E_INVALID, "dit_pack_layout: segment %d cond_row=%d", i, segs[i].cond_row);
    total += n;
    if (total >= (int64_t(1) << 31))
      return set_error(DIT_E_INVALID, "dit_pack_layout: more than 2^31-1 tokens");
    cu_seqlens[i + 1] = static_cast<int32_t>(total);
  }
  for (int i = 0; i < n_segs; ++i) {
    for (int32_t r = cu_seqlens[i]; r < cu_seqlens[i + 1]; ++r) {
      if (cond_idx) cond_idx[r] = segs[i].cond_row;
      if (doc_id) doc_id[r] = i;
    }
  }
  *n_tokens = static_cast<int>(total);
  return DIT_OK;
}

// Page "stream the ORIGINAL bf16 DiT to the device", section "What this
// enables": the cos/sin tables are built on the host before any kernel.  Page
// "port the MiniMax-H3 omni-modal video+audio DiT", update "video-VAE ViT3D
// decoder complete": per-axis frequency blocks are concatenated, and the
// rotate_half pairing (i, i + rot/2) tiles the concatenation twice; a
// DIT_ROPE_CENTERED modality takes its angles from cell centres of [-1, 1)
// scaled by 2 pi (the same update's length-normalized token ids).
extern "C" int dit_rope_cache_build(const dit_config* cfg, const dit_segment* segs, int n_segs,
                                    float* cos_host, float* sin_host) {
  if (cfg == nullptr || segs == nullptr || cos_host == nullptr || sin_host == nullptr)
    return set_error(DIT_E_INVALID, "dit_rope_cache_build: null argument");
  const int half = cfg->rot_dim / 2;
  // Frequency table per modality: the concatenation over axes of inv_freq_a.
  std::vector<std::vector<double>> freq(cfg->n_mod);
  std::vector<std::vector<int>> axis_of(cfg->n_mod);
  for (int m = 0; m < cfg->n_mod; ++m) {
    const dit_modality& md = cfg->mod[m];
    for (int a = 0; a < md.n_axes; ++a) {
      const int da = md.axis_dim[a];
      for (int j = 0; j < da / 2; ++j) {
        const double e = static_cast<double>(2 * j) / static_cast<double>(da);
        freq[m].push_back(1.0 / std::pow(cfg->theta, e));
        axis_of[m].push_back(a);
      }
    }
    if (static_cast<int>(freq[m].size()) != half)
      return set_error(DIT_E_INVALID, "dit_rope_cache_build: modality %d axis dims do not sum to rot_dim", m);
  }
  int64_t row = 0;
  for (int i = 0; i < n_segs; ++i) {
    const dit_segment& s = segs[i];
    int64_t n;
    if (segment_tokens(cfg, s, &n) != 0)
      return set_error(DIT_E_INVALID, "dit_rope_cache_build: segment %d is malformed", i);
    const int axes = cfg->mod[s.modality].n_axes;
    const std::vector<double>& f = freq[s.modality];
    const std::vector<int>& ax = axis_of[s.modality];
    for (int64_t t = 0; t < n; ++t, ++row) {
      int64_t pos[3] = {t, 0, 0};
      if (axes == 3) {
        pos[2] = t % s.grid[2];
        pos[1] = (t / s.grid[2]) % s.grid[1];
        pos[0] = t / (static_cast<int64_t>(s.grid[2]) * s.grid[1]);
      }
      float* cr = cos_host + row * half;
      float* sr = sin_host + row * half;
      const bool centered = cfg->mod[s.modality].rope_grid == DIT_ROPE_CENTERED;
      for (int j = 0; j < half; ++j) {
        double ang;
        if (centered) {
          // the centre of cell pos of [-1, 1) split in the axis' extent, times 2 pi
          const double c = (2.0 * static_cast<double>(pos[ax[j]]) + 1.0) / static_cast<double>(s.grid[ax[j]]) - 1.0;
          ang = (2.0 * M_PI * c) * f[j];
        } else {
          ang = static_cast<double>(pos[ax[j]]) * f[j];
        }
        cr[j] = static_cast<float>(std::cos(ang));
        sr[j] = static_cast<float>(std::sin(ang));
      }
    }
  }
  return DIT_OK;
}

extern "C" int dit_timestep_embedding(const float* t_host, int n, int dim, float* out_host) {
  if (t_host == nullptr || out_host == nullptr || n < 0 || dim <= 0 || dim % 2)
    return set_error(DIT_E_INVALID, "dit_timestep_embedding: bad argument (dim must be even)");
  const int h = dim / 2;
  for (int i = 0; i < n; ++i) {
    const double t = static_cast<double>(t_host[i]);
    for (int j = 0; j < h; ++j) {
      const double f = std::pow(10000.0, -static_cast<double>(j) / static_cast<double>(h));
      const double a = t * f;
      out_host[static_cast<int64_t>(i) * dim + j] = static_cast<float>(std::cos(a));
      out_host[static_cast<int64_t>(i) * dim + h + j] = static_cast<float>(std::sin(a));
    }
  }
  return DIT_OK;
}

// Page "port the MiniMax-H3 omni-modal video+audio DiT", update "quantized
// arms land" item 2: the rectified-flow time-shift sigma schedule (video shift
// 12, audio shift 3).
extern "C" int dit_sigma_schedule(double shift, int n_steps, double* sigma_host, float* dt_host) {
  if (n_steps < 1 || !(shift > 0.0 && std::isfinite(shift)))
    return set_error(DIT_E_INVALID, "dit_sigma_schedule: n_steps must be >= 1 and shift positive and finite");
  std::vector<double> sig(n_steps + 1);
  for (int i = 0; i <= n_steps; ++i) {
    const double s = 1.0 - static_cast<double>(i) / static_cast<double>(n_steps);
    sig[i] = shift * s / (1.0 + (shift - 1.0) * s);
  }
  if (sigma_host) std::memcpy(sigma_host, sig.data(), sizeof(double) * (n_steps + 1));
  if (dt_host)
    for (int i = 0; i < n_steps; ++i) dt_host[i] = static_cast<float>(sig[i + 1] - sig[i]);
  return DIT_OK;
}

// ---------------------------------------------------------------- int8 slices of fp32 weights
// The staging-time twin of the device slicing (slice_rows): per row, e with
// max|x| < 2^e (frexp), then five truncating 7-bit digits of x 2^-e; five
// planes of [Kp/32][R][32] int8 (zero past K), then R int32 exponents 256
// bytes further aligned.  All steps are exact in fp32, so both sides produce
// the same bytes.  A weight row holding a NaN or an Inf has no slicing (the
// device marks such activation rows instead): the first one is returned.
namespace dit {
int64_t host_slice_rows(int64_t R, int64_t K, int64_t Kp, const float* X, int8_t* out) {
  const size_t plane = static_cast<size_t>(R) * Kp;
  int32_t* E = reinterpret_cast<int32_t*>(out + ((5 * plane + 255) & ~size_t(255)));
  for (int64_t r = 0; r < R; ++r) {
    const float* x = X + r * K;
    float mx = 0.f;
    for (int64_t k = 0; k < K; ++k) {
      if (!std::isfinite(x[k])) return r;
      mx = std::fmax(mx, std::fabs(x[k]));
    }
    int e = 0;
    if (mx > 0.f) std::frexp(mx, &e);
    E[r] = e;
    for (int64_t k = 0; k < Kp; ++k) {
      float f = k < K ? std::ldexp(x[k], -e) : 0.f;
      for (int s = 0; s < 5; ++s) {
        f *= 128.f;
        const float d = std::trunc(f);
        f -= d;
        out[s * plane + (static_cast<size_t>(k / 32) * R + r) * 32 + (k % 32)] = static_cast<int8_t>(static_cast<int>(d));
      }
    }
  }
  return -1;
}

// ---------------------------------------------------------------- MXFP8 weights
// The staging-time twin of the device quantizer (mx8.hip): per 32 consecutive
// K values, the smallest power-of-two scale 2^s with max|v| <= 448 2^s (E8M0
// byte s + 127; byte 0 for an all-zero block), then each v 2^-s rounded to
// nearest-even E4M3 (sign kept).  Every step is exact in float, so both sides
// produce the same bytes.
static uint8_t host_e4m3(float y) {
  const uint8_t sgn = std::signbit(y) ? 0x80 : 0;
  const float a = std::fabs(y);
  if (a >= 448.0f) return sgn | 0x7E;
  if (a < 0.015625f) return sgn | static_cast<uint8_t>(std::nearbyint(a * 512.0f));
  uint32_t ua;
  std::memcpy(&ua, &a, 4);
  int e = static_cast<int>(ua >> 23) - 127;
  uint32_t keep = (ua >> 20) & 7u;
  const uint32_t rem = ua & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0;
    ++e;
  }
  return sgn | static_cast<uint8_t>((static_cast<uint32_t>(e + 7) << 3) | keep);
}

static int64_t quantize_mx8_rows(int64_t r0, int64_t r1, int64_t K, const float* X, uint8_t* codes, uint8_t* scales) {
  const int64_t kb = K / 32;
  for (int64_t r = r0; r < r1; ++r) {
    for (int64_t b = 0; b < kb; ++b) {
      const float* v = X + r * K + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        if (!std::isfinite(v[i])) return r;
        amax = std::fmax(amax, std::fabs(v[i]));
      }
      int s = 0;
      uint8_t byte = 0;
      if (amax > 0.0f) {
        int ef;
        const float f = std::frexp(amax, &ef);
        s = ef - 1 - 8 + (f > 0.875f ? 1 : 0);
        s = s < -127 ? -127 : (s > 127 ? 127 : s);
        byte = static_cast<uint8_t>(s + 127);
      }
      scales[r * kb + b] = byte;
      for (int i = 0; i < 32; ++i) codes[r * K + b * 32 + i] = host_e4m3(std::ldexp(v[i], -s));
    }
  }
  return -1;
}

// ---------------------------------------------------------------- MXFP4 weights
// The staging-time MXFP4 quantizer: per 32 consecutive K values, the smallest
// power-of-two scale 2^s with max|v| <= 6 2^s (E8M0 byte s + 127; byte 0 for
// an all-zero block), then v 2^-s rounded to the nearest OCP FP4 E2M1 value
// (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the even mantissa bit, the
// sign kept; two codes per byte, the one at even K in the low nibble.  Every
// step is exact in float.
static uint8_t host_e2m1(float y) {
  const float a = std::fabs(y);
  int m;
  if (a >= 6.0f) {
    m = 7;
  } else if (a < 1.0f) {
    m = static_cast<int>(std::nearbyint(a * 2.0f));  // steps of 0.5: codes 0, 1 and 2 (= 1.0)
  } else {
    int e;
    const float f = std::frexp(a, &e);  // a = 2f 2^(e-1), 2f in [1, 2)
    int q = static_cast<int>(std::nearbyint((2.0f * f - 1.0f) * 2.0f));
    int b = e - 1;
    if (q == 2) {
      q = 0;
      ++b;
    }
    m = ((b + 1) << 1) | q;
  }
  return static_cast<uint8_t>((std::signbit(y) ? 8 : 0) | m);
}

static int64_t quantize_mx4_rows(int64_t r0, int64_t r1, int64_t K, const float* X, uint8_t* codes, uint8_t* scales) {
  const int64_t kb = K / 32;
  for (int64_t r = r0; r < r1; ++r) {
    for (int64_t b = 0; b < kb; ++b) {
      const float* v = X + r * K + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        if (!std::isfinite(v[i])) return r;
        amax = std::fmax(amax, std::fabs(v[i]));
      }
      int s = 0;
      uint8_t byte = 0;
      if (amax > 0.0f) {
        int ef;
        const float f = std::frexp(amax, &ef);
        s = ef - 1 - 2 + (f > 0.75f ? 1 : 0);
        s = s < -127 ? -127 : (s > 127 ? 127 : s);
        byte = static_cast<uint8_t>(s + 127);
      }
      scales[r * kb + b] = byte;
      uint8_t* c = codes + r * (K / 2) + b * 16;
      for (int i = 0; i < 16; ++i)
        c[i] = static_cast<uint8_t>(host_e2m1(std::ldexp(v[2 * i], -s)) | (host_e2m1(std::ldexp(v[2 * i + 1], -s)) << 4));
    }
  }
  return -1;
}

// Rows in parallel over the host's cores (each row is independent; the
// result does not depend on the split).
template <typename RowFn>
static int64_t quantize_rows_parallel(int64_t R, int64_t K, RowFn rows) {
  unsigned nt = std::thread::hardware_concurrency();
  nt = nt == 0 ? 1 : (nt > 16 ? 16 : nt);
  if (R * K < (int64_t(1) << 22) || nt == 1) return rows(0, R);
  std::vector<int64_t> bad(nt, -1);
  std::vector<std::thread> pool;
  const int64_t per = (R + nt - 1) / nt;
  for (unsigned t = 0; t < nt; ++t) {
    const int64_t r0 = per * t, r1 = r0 + per < R ? r0 + per : R;
    if (r0 >= r1) break;
    pool.emplace_back([=, &bad] { bad[t] = rows(r0, r1); });
  }
  for (auto& th : pool) th.join();
  for (int64_t b : bad)
    if (b >= 0) return b;  // threads cover rows in order: the first one found is the smallest
  return -1;
}

int64_t host_quantize_mx8(int64_t R, int64_t K, const float* X, uint8_t* codes, uint8_t* scales) {
  return quantize_rows_parallel(R, K, [=](int64_t r0, int64_t r1) { return quantize_mx8_rows(r0, r1, K, X, codes, scales); });
}

int64_t host_quantize_mx4(int64_t R, int64_t K, const float* X, uint8_t* codes, uint8_t* scales) {
  return quantize_rows_parallel(R, K, [=](int64_t r0, int64_t r1) { return quantize_mx4_rows(r0, r1, K, X, codes, scales); });
}

}  // namespace dit

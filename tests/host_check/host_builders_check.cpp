// Host-side checker of the library's table builders, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitized.py (plain g++, no
// HIP).  It runs the builders on the configurations in a request file and
// writes their outputs, raw, to a result file that the test compares with the
// shipped library's.
//
// Request file (native-endian, written by the test):
//   int32 n_cases; then per case:
//     dit_config (raw struct); int32 n_segs; dit_segment[n_segs] (raw structs)
//   int32 n_t; float t[n_t]; int32 dim
//   int32 n_shift; double shift[n_shift]; int32 n_steps
//   int64 R, K; float X[R*K]
// Result file: per case int32 rc, then (rc == 0) int32 N, cu[n_segs+1],
// cond[N], doc[N], cos[N*rot/2], sin[N*rot/2]; then the embedding [n_t*dim]
// float, per shift sigma [n_steps+1] double and dt [n_steps] float; then the
// slices of X (5*R*Kp int8 + 256-aligned int32 exponents) and the int64 result
// of host_slice_rows.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "dit.h"
#include "internal.h"

namespace dit {
int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace dit

template <typename T>
static T rd(FILE* f) {
  T v;
  if (fread(&v, sizeof(T), 1, f) != 1) { fprintf(stderr, "short request\n"); exit(2); }
  return v;
}
template <typename T>
static void rdn(FILE* f, T* p, size_t n) {
  if (n && fread(p, sizeof(T), n, f) != n) { fprintf(stderr, "short request\n"); exit(2); }
}
template <typename T>
static void wr(FILE* f, const T* p, size_t n) { fwrite(p, sizeof(T), n, f); }

int main(int argc, char** argv) {
  if (argc != 3) { fprintf(stderr, "usage: %s request result\n", argv[0]); return 2; }
  FILE* in = fopen(argv[1], "rb");
  FILE* out = fopen(argv[2], "wb");
  if (!in || !out) return 2;
  const int n_cases = rd<int32_t>(in);
  for (int c = 0; c < n_cases; ++c) {
    const dit_config cfg = rd<dit_config>(in);
    const int n_segs = rd<int32_t>(in);
    std::vector<dit_segment> segs(n_segs > 0 ? n_segs : 0);
    rdn(in, segs.data(), segs.size());
    int N = 0;
    std::vector<int32_t> cu(segs.size() + 1);
    int32_t rc = dit_pack_layout(&cfg, segs.data(), n_segs, cu.data(), nullptr, nullptr, &N);
    std::vector<int32_t> cond, doc;
    std::vector<float> cs, sn;
    if (rc == DIT_OK) {
      cond.resize(N);
      doc.resize(N);
      rc = dit_pack_layout(&cfg, segs.data(), n_segs, cu.data(), cond.data(), doc.data(), &N);
    }
    if (rc == DIT_OK) {
      const size_t half = static_cast<size_t>(cfg.rot_dim / 2);
      cs.resize(static_cast<size_t>(N) * half);
      sn.resize(cs.size());
      rc = dit_rope_cache_build(&cfg, segs.data(), n_segs, cs.data(), sn.data());
    }
    wr(out, &rc, 1);
    if (rc == DIT_OK) {
      int32_t n32 = N;
      wr(out, &n32, 1);
      wr(out, cu.data(), cu.size());
      wr(out, cond.data(), cond.size());
      wr(out, doc.data(), doc.size());
      wr(out, cs.data(), cs.size());
      wr(out, sn.data(), sn.size());
    }
  }
  const int n_t = rd<int32_t>(in);
  std::vector<float> t(n_t);
  rdn(in, t.data(), t.size());
  const int dim = rd<int32_t>(in);
  std::vector<float> emb(static_cast<size_t>(n_t) * dim);
  if (dit_timestep_embedding(t.data(), n_t, dim, emb.data()) != DIT_OK) return 3;
  wr(out, emb.data(), emb.size());
  const int n_shift = rd<int32_t>(in);
  std::vector<double> shifts(n_shift);
  rdn(in, shifts.data(), shifts.size());
  const int n_steps = rd<int32_t>(in);
  for (double sh : shifts) {
    std::vector<double> sig(n_steps + 1);
    std::vector<float> dt(n_steps);
    if (dit_sigma_schedule(sh, n_steps, sig.data(), dt.data()) != DIT_OK) return 4;
    wr(out, sig.data(), sig.size());
    wr(out, dt.data(), dt.size());
  }
  // error paths, for the sanitizers only
  if (dit_sigma_schedule(0.0, n_steps, nullptr, nullptr) == DIT_OK) return 5;
  if (dit_timestep_embedding(t.data(), n_t, 3, emb.data()) == DIT_OK) return 6;
  const int64_t R = rd<int64_t>(in), K = rd<int64_t>(in);
  std::vector<float> X(static_cast<size_t>(R * K));
  rdn(in, X.data(), X.size());
  const int64_t Kp = (K + 31) / 32 * 32;
  const size_t plane = static_cast<size_t>(R * Kp);
  std::vector<int8_t> sl(((5 * plane + 255) & ~size_t(255)) + sizeof(int32_t) * static_cast<size_t>(R));
  const int64_t bad = dit::host_slice_rows(R, K, Kp, X.data(), sl.data());
  wr(out, sl.data(), sl.size());
  wr(out, &bad, 1);
  fclose(out);
  fclose(in);
  return 0;
}

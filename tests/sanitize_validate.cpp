// Drives the library's host-only checks (hga_validate.cpp) over many shapes,
// for the CPU tests' address- and undefined-behaviour-sanitized build: every
// field takes ordinary, boundary and extreme values (seeded), and each
// accepted shape is checked against the limits the header states.
#include <climits>
#include <cstdio>
#include <cstring>

#include "hga.h"

namespace {

unsigned long long state = 0x9E3779B97F4A7C15ull;
unsigned long long next() {   // SplitMix64
  unsigned long long z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int pick(int n) { return (int)(next() % (unsigned long long)n); }

int value() {
  static const int special[] = {0, 1, -1, 2, 7, 8, 63, 64, 65, 128, 192, 512, 513, 1024,
                                2048, 16384, 65536, 131072, 131073, 262144, 1 << 23,
                                1 << 30, INT_MAX, INT_MIN, INT_MAX - 63, -64};
  if (pick(3) == 0) return special[pick((int)(sizeof(special) / sizeof(special[0])))];
  if (pick(2) == 0) return 64 * (1 + pick(2048));
  return pick(1 << 20) - (1 << 10);
}

int fails = 0;
void expect(bool ok, const char* what, const hga_shape& s) {
  if (ok) return;
  ++fails;
  std::printf("violated: %s (B=%d Hq=%d Hkv=%d D=%d q=%d kv=%d k=%d g=%d cap=%d)\n", what,
              s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.q_len, s.kv_len, s.top_k,
              s.top_g, s.kv_capacity);
}

}  // namespace

int main() {
  int accepted = 0, accepted_decode = 0;
  for (int it = 0; it < 200000; ++it) {
    hga_shape s;
    s.batch = pick(4) ? 1 + pick(16) : value();
    s.n_kv_heads = pick(4) ? 1 + pick(8) : value();
    s.n_q_heads = pick(4) ? (int)((unsigned)s.n_kv_heads * (unsigned)(1 + pick(8))) : value();
    s.head_dim = pick(3) ? (pick(2) ? 64 : 128) : value();
    s.q_len = pick(4) ? 64 * (1 + pick(64)) : value();
    s.kv_len = pick(4) ? (int)((unsigned)s.q_len + 64u * (unsigned)pick(2048)) : value();
    s.top_k = pick(4) ? pick(70) : value();
    s.top_g = pick(4) ? pick(600) : value();
    const unsigned bits[] = {0x3DB504F3u, 0u, 0x7F800000u, 0x7FC00000u, 0xFF800000u, 0xBF800000u};
    unsigned b = bits[pick(6)];
    std::memcpy(&s.softmax_scale, &b, sizeof(b));
    s.dtype = pick(8) ? pick(2) : value();
    s.kv_capacity = pick(2) ? 0 : (pick(2) ? (int)((unsigned)s.kv_len + 64u * (unsigned)pick(64))
                                           : value());
    if (hga_validate_shape(&s) == HGA_OK) {
      ++accepted;
      expect(s.batch >= 1 && s.n_kv_heads >= 1 && s.n_q_heads % s.n_kv_heads == 0, "heads", s);
      expect(s.q_len >= 64 && s.q_len % 64 == 0 && s.q_len <= s.kv_len, "q_len", s);
      expect(s.kv_len % 64 == 0 && s.kv_len <= HGA_MAX_KV_LEN, "kv_len", s);
      expect(s.top_k >= 0 && s.top_k <= HGA_MAX_TOP_K && s.top_g >= 0 &&
                 s.top_g <= HGA_MAX_TOP_G, "budgets", s);
      expect(s.head_dim == 64 || s.head_dim == 128, "head_dim", s);
      const int g = hga_stage_min_groups(&s);
      expect(g >= 0 && g % 8 == 0 && g <= 8 * ((s.kv_len - s.q_len) / 64) + 7, "stage", s);
    }
    hga_shape d = s;
    d.q_len = 1;
    d.kv_len = pick(4) ? 1 + pick(131072) : value();
    if (hga_validate_decode_shape(&d) == HGA_OK) {
      ++accepted_decode;
      const int cap = d.kv_capacity > 0 ? d.kv_capacity : d.kv_len;
      expect(cap % 64 == 0 && cap >= d.kv_len && cap <= HGA_MAX_KV_LEN, "decode capacity", d);
    }
    (void)hga_status_str((hga_status)pick(8));
  }
  expect(hga_validate_shape(nullptr) == HGA_ERR_NULL, "null", hga_shape{});
  expect(hga_stage_min_groups(nullptr) == -1, "null stage", hga_shape{});
  std::printf("accepted %d block shapes and %d decode shapes; %d violations\n", accepted,
              accepted_decode, fails);
  return fails == 0 && accepted > 1000 && accepted_decode > 1000 ? 0 : 1;
}

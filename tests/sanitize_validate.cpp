// Drives the library's host-only checks (hga_validate.cpp, and the workspace
// layouts and staging checks of hga_layout.h) over many shapes, for the CPU
// tests' address- and undefined-behaviour-sanitized build: every field takes
// ordinary, boundary and extreme values (seeded), and each accepted shape or
// argument set is checked against the limits the header states, with sizes
// recomputed in 128-bit arithmetic.
#include <climits>
#include <cstdio>
#include <cstring>

#include "hga.h"
#include "hga_layout.h"

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

typedef unsigned __int128 u128;
u128 up256(u128 n) { return (n + 255) / 256 * 256; }

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
  int accepted = 0, accepted_decode = 0, staged = 0, staged_prev = 0;
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
      // backward workspace: the three parts, each rounded, recomputed wide
      size_t ws = 0;
      expect(hga_attend_bwd_workspace(&s, &ws) == HGA_OK, "bwd workspace ok", s);
      const u128 B = (u128)s.batch, Hq = (u128)s.n_q_heads, Hkv = (u128)s.n_kv_heads;
      const u128 want = up256(B * Hq * (u128)s.q_len * 4) +
                        up256(B * Hq * (u128)(s.q_len / 64) * (u128)(s.kv_len / 64)) +
                        2 * up256(B * Hkv * (u128)(s.kv_len / 64) * 4);
      expect((u128)ws == want, "bwd workspace size", s);
      expect(hga_attend_bwd_workspace(&s, nullptr) == HGA_ERR_NULL, "bwd workspace null", s);
      // staging: sizes and argument checks over ordinary and extreme values
      const int sg = pick(2) ? g + 8 * pick(64) : (pick(2) ? 8 * pick(2049) : value());
      size_t sb = 0;
      const hga_status sst = hga_stage_workspace(&s, sg, &sb);
      const bool sg_ok = sg >= 0 && sg % 8 == 0 && sg <= HGA_MAX_KV_LEN / 8;
      expect((sst == HGA_OK) == sg_ok, "stage workspace accepts", s);
      if (sst == HGA_OK)
        expect((u128)sb == 2 * up256(B * Hkv * (u128)sg * 4) + up256(B * Hkv * 4),
               "stage workspace size", s);
      const long long capw = (8LL * sg + s.q_len + 63) / 64 * 64 + 64 * pick(4);
      const int cap = pick(2) && capw <= HGA_MAX_KV_LEN ? (int)capw
                                                         : (pick(3) ? 64 * (pick(2049) + 1) : value());
      hga_stage_prev pv;
      std::memset(&pv, 0, sizeof(pv));
      char dummy[16];
      pv.K_stage = pick(8) ? dummy : nullptr;
      pv.V_stage = dummy;
      pv.workspace = dummy;
      pv.stage_groups = pick(3) ? 8 * pick(2049) : value();
      pv.stage_capacity = pick(3) ? 64 * (pick(2049) + 1) : value();
      pv.q0 = pick(3) ? 64 * pick(2048) : value();
      pv.q_len = pick(3) ? 64 * (pick(64) + 1) : value();
      pv.workspace_bytes = pick(4) ? (size_t)pick(1 << 30) : (size_t)-1 >> pick(64);
      const int q0s = s.kv_len - s.q_len;
      if (pick(2) && q0s >= 64) {
        // a consistent previous staging: an earlier segment of the history
        pv.q_len = 64 * (1 + pick(q0s / 64 < 64 ? q0s / 64 : 64));
        pv.q0 = 64 * pick((q0s - pv.q_len) / 64 + 1);
        pv.stage_groups = 8 * pick(2049);
        const long long pc = (8LL * pv.stage_groups + pv.q_len + 63) / 64 * 64 + 64 * pick(4);
        pv.stage_capacity = pc <= HGA_MAX_KV_LEN ? (int)pc : HGA_MAX_KV_LEN;
        const u128 need = up256((u128)s.batch * (u128)s.n_kv_heads * (u128)pv.stage_groups * 4) +
                          up256((u128)s.batch * (u128)s.n_kv_heads * 4);
        pv.workspace_bytes = pick(8) ? (size_t)need + (size_t)pick(512) : (size_t)need - 1;
      }
      const hga_stage_prev* pp = pick(2) ? &pv : nullptr;
      const hga_status cst = hga_layout::check_stage_args(&s, sg, cap, pp);
      if (cst == HGA_OK) {
        ++(pp ? staged_prev : staged);
        expect(sg % 8 == 0 && sg >= g && sg <= HGA_MAX_KV_LEN / 8, "stage groups", s);
        expect(cap % 64 == 0 && cap <= HGA_MAX_KV_LEN && (long long)cap >= 8LL * sg + s.q_len,
               "stage capacity", s);
        if (pp) {
          const long long q0 = s.kv_len - s.q_len;
          expect(pv.K_stage && pv.V_stage && pv.workspace, "prev pointers", s);
          expect(pv.stage_groups >= 0 && pv.stage_groups % 8 == 0 &&
                     pv.stage_groups <= HGA_MAX_KV_LEN / 8 && pv.q0 >= 0 && pv.q0 % 64 == 0 &&
                     pv.q_len >= 64 && pv.q_len % 64 == 0 && pv.q0 + (long long)pv.q_len <= q0 &&
                     pv.stage_capacity % 64 == 0 && pv.stage_capacity <= HGA_MAX_KV_LEN &&
                     (long long)pv.stage_capacity >= 8LL * pv.stage_groups + pv.q_len,
                 "prev geometry", s);
          expect((u128)pv.workspace_bytes >=
                     up256(B * Hkv * (u128)pv.stage_groups * 4) + up256(B * Hkv * 4),
                 "prev workspace", s);
        }
      }
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
  size_t nb = 0;
  expect(hga_attend_bwd_workspace(nullptr, &nb) == HGA_ERR_NULL, "null bwd workspace", hga_shape{});
  expect(hga_stage_workspace(nullptr, 8, &nb) == HGA_ERR_NULL, "null stage workspace", hga_shape{});
  std::printf("accepted %d block shapes, %d decode shapes, %d staging argument sets and %d "
              "with a previous staging; %d violations\n",
              accepted, accepted_decode, staged, staged_prev, fails);
  return fails == 0 && accepted > 1000 && accepted_decode > 1000 && staged > 100 &&
                 staged_prev > 100
             ? 0
             : 1;
}

/*
 * HGA CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64, single-threaded implementation of Hierarchical Global
 * Attention (HGA) as described on the page "BMW's 16 GB GPU just did what needs
 * an A100" (seventnews.com, English edition), section "What HGA does
 * differently".  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no code, header, table or helper
 * with the HIP library; the two never include or call each other.
 *
 * Everything is plain nested loops in double precision, summed sequentially in
 * index order, so that each step can be checked against the page by eye.  The
 * chunk size C and group size G are parameters (the page fixes 64 and 8) so
 * that hand-made cases can use smaller ones.  The query block size equals C.
 *
 * Layouts (row-major, contiguous):
 *   Q, O, dO, dQ : [B][Hq][Sq][D]      K, V, dK, dV : [B][Hkv][Skv][D]
 *   lse          : [B][Hq][Sq]         chunk_mean   : [B][Hkv][Skv/C][D]
 *   group_mean   : [B][Hkv][Skv/G][D]
 *   chunk_idx    : [B][Hq][Sq/C][top_k]  group_idx : [B][Hq][Sq/C][top_g]
 * The Sq queries are the LAST Sq positions of the Skv-long sequence
 * (q0 = Skv - Sq): a segment at the end of its history.
 *
 * Return codes: 0 ok, 2 bad shape, 3 invalid routing indices, 4 non-finite input.
 *
 * Readings taken where the page is silent:
 *  - summary of a chunk (and of a group) = mean of its keys;
 *  - the query side of the routing score = mean of the block's C queries
 *    (strictly causal variant: mean of the C queries before the block);
 *  - score = plain dot product; routing is per query head; a GQA query head hq
 *    reads kv head hq / (Hq/Hkv);
 *  - candidates are the chunks strictly before the query block's own chunk;
 *    the block's own chunk is always attended, causally;
 *  - top-g is taken jointly over all groups of the kept chunks;
 *  - order is (score descending, index ascending); kept indices are emitted in
 *    ascending order and padded with -1;
 *  - softmax scale 1/sqrt(D) unless given; lse in natural log;
 *  - the backward holds the routing fixed (no gradient through selection);
 *  - decode (one new token at the end of an L-token cache) is the block form
 *    with a block of one query: the routing query is that query, the
 *    candidates are the complete chunks before its own chunk (L-1)/C, and the
 *    own chunk is attended from its start up to the query.
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <utility>
#include <vector>

namespace {

inline long long idx4(int a, int b, int c, int d, int B_, int C_, int D_) {
  return (((long long)a * B_ + b) * C_ + c) * D_ + d;
}

bool all_finite(const double* x, long long n) {
  for (long long i = 0; i < n; ++i)
    if (!std::isfinite(x[i])) return false;
  return true;
}

bool shape_ok(int B, int Hq, int Hkv, int Sq, int Skv, int D, int C, int G) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || C <= 0 || G <= 0) return false;
  if (Hq % Hkv != 0) return false;
  if (C % G != 0) return false;
  if (Sq <= 0 || Skv <= 0 || Sq > Skv) return false;
  if (Sq % C != 0 || Skv % C != 0) return false;
  return true;
}

/* Orders candidates by (score descending, index ascending).  -0.0 and +0.0
 * compare equal under IEEE ==, so they are ties broken by index. */
bool better(const std::pair<double, int>& a, const std::pair<double, int>& b) {
  if (a.first > b.first) return true;
  if (a.first < b.first) return false;
  return a.second < b.second;
}

/* Keeps the best min(keep, n) candidates and returns their indices ascending. */
std::vector<int> top_by_score(std::vector<std::pair<double, int>> cand, int keep) {
  std::sort(cand.begin(), cand.end(), better);
  int n = std::min<int>(keep, (int)cand.size());
  std::vector<int> out;
  for (int i = 0; i < n; ++i) out.push_back(cand[i].second);
  std::sort(out.begin(), out.end());
  return out;
}

/* The exact key positions attended by the query at absolute position p of a
 * query block whose own chunk is cb: every token of every kept group, then the
 * own chunk's tokens from its start up to and including p (causal). */
std::vector<int> key_set(const int32_t* groups, int top_g, int G, int C, int cb, int p) {
  std::vector<int> keys;
  for (int i = 0; i < top_g; ++i) {
    int gam = groups[i];
    if (gam < 0) continue;
    for (int t = 0; t < G; ++t) keys.push_back(gam * G + t);
  }
  for (int j = cb * C; j <= p; ++j) keys.push_back(j);
  return keys;
}

/* Checks a routing row: valid entries strictly ascending, all before the own
 * chunk, -1 only as trailing padding. */
bool groups_valid(const int32_t* groups, int top_g, int G, int C, int cb) {
  int prev = -1;
  bool pad = false;
  for (int i = 0; i < top_g; ++i) {
    int gam = groups[i];
    if (gam < 0) {
      if (gam != -1) return false;
      pad = true;
      continue;
    }
    if (pad) return false;
    if (gam <= prev) return false;
    if ((long long)(gam + 1) * G > (long long)cb * C) return false;
    prev = gam;
  }
  return true;
}

}  // namespace

extern "C" {

int hgao_version(void) { return 1; }

/* Chunk and group summaries.  The page keeps a compact summary vector per
 * 64-token chunk resident in GPU memory; it gives no formula, so the summary is
 * taken to be the mean of the chunk's keys, and the group summary (used when a
 * kept chunk is opened at the 8-token group level) the mean of the group's keys. */
int hgao_summaries(int B, int Hkv, int S, int D, int C, int G, const double* K,
                   double* chunk_mean, double* group_mean) {
  if (B <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || C <= 0 || G <= 0) return 2;
  if (S % C != 0 || S % G != 0) return 2;
  if (!all_finite(K, (long long)B * Hkv * S * D)) return 4;
  const int nc = S / C, ng = S / G;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hkv; ++h) {
      for (int c = 0; c < nc; ++c)
        for (int d = 0; d < D; ++d) {
          double s = 0.0;
          for (int j = c * C; j < c * C + C; ++j) s += K[idx4(b, h, j, d, Hkv, S, D)];
          chunk_mean[idx4(b, h, c, d, Hkv, nc, D)] = s / C;
        }
      for (int g = 0; g < ng; ++g)
        for (int d = 0; d < D; ++d) {
          double s = 0.0;
          for (int j = g * G; j < g * G + G; ++j) s += K[idx4(b, h, j, d, Hkv, S, D)];
          group_mean[idx4(b, h, g, d, Hkv, ng, D)] = s / G;
        }
    }
  return 0;
}

/* Two-level routing (page section "What HGA does differently"): for every
 * query block the block query scores the chunk summaries of the history and
 * keeps the top_k chunks; it then opens those chunks at the 8-token group level,
 * scores their group summaries and keeps the top_g groups.
 *
 * forced_chunk_idx (nullable, [B][Hq][Sq/C][top_k], ascending, -1 padded):
 * when given, the chunk stage is skipped and these chunk sets are opened
 * instead (used to re-derive the group choice for a given chunk set).
 * chunk_score / group_score (nullable, [B][Hq][Sq/C][Skv/C] and
 * [B][Hq][Sq/C][Skv/G]): the fp64 scores of every candidate, NaN elsewhere. */
/* Routing of every query block.  The block query is the mean of the block's C
 * query vectors; with `causal` it is the mean of the C query vectors just
 * before the block instead (the previous block of Q, or for the first block of
 * a segment the C rows of Qprev [B][Hq][C][D]), so that no position's routing
 * depends on a later position (page section "The one real caveat: causal
 * leakage": a block's routing mixes several of its query positions). */
static int route_impl(int B, int Hq, int Hkv, int Sq, int Skv, int D, int C, int G,
                      int top_k, int top_g, const double* Q, bool causal, const double* Qprev,
                      const double* chunk_mean, const double* group_mean,
                      const int32_t* forced_chunk_idx, int32_t* chunk_idx, int32_t* group_idx,
                      double* chunk_score, double* group_score) {
  if (!shape_ok(B, Hq, Hkv, Sq, Skv, D, C, G) || top_k < 0 || top_g < 0) return 2;
  if (!all_finite(Q, (long long)B * Hq * Sq * D)) return 4;
  const int r = Hq / Hkv, nblk = Sq / C, nc = Skv / C, ng = Skv / G, gpc = C / G;
  const int q0 = Skv - Sq;
  if (causal && q0 > 0 && (top_k > 0 || top_g > 0)) {
    if (!Qprev) return 2;
    if (!all_finite(Qprev, (long long)B * Hq * C * D)) return 4;
  }
  const double nan = std::nan("");
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq) {
      const int hkv = hq / r;
      for (int blk = 0; blk < nblk; ++blk) {
        const long long row = ((long long)b * Hq + hq) * nblk + blk;
        const int cb = q0 / C + blk; /* the block's own chunk */

        /* block query: mean of C query vectors (the block's own, or with
         * `causal` the C vectors before the block); unused without candidates */
        std::vector<double> qbar(D, 0.0);
        if (cb > 0) {
          for (int d = 0; d < D; ++d) {
            double s = 0.0;
            for (int i = 0; i < C; ++i) {
              if (!causal)
                s += Q[idx4(b, hq, blk * C + i, d, Hq, Sq, D)];
              else if (blk > 0)
                s += Q[idx4(b, hq, (blk - 1) * C + i, d, Hq, Sq, D)];
              else
                s += Qprev[idx4(b, hq, i, d, Hq, C, D)];
            }
            qbar[d] = s / C;
          }
        }

        /* chunk stage: candidates are the chunks strictly before cb */
        std::vector<int> kept_chunks;
        if (chunk_score)
          for (int c = 0; c < nc; ++c) chunk_score[row * nc + c] = nan;
        std::vector<std::pair<double, int>> cand;
        for (int c = 0; c < cb; ++c) {
          double s = 0.0;
          for (int d = 0; d < D; ++d) s += qbar[d] * chunk_mean[idx4(b, hkv, c, d, Hkv, nc, D)];
          cand.push_back({s, c});
          if (chunk_score) chunk_score[row * nc + c] = s;
        }
        if (forced_chunk_idx) {
          for (int i = 0; i < top_k; ++i) {
            int c = forced_chunk_idx[row * top_k + i];
            if (c < 0) continue;
            if (c >= cb) return 3;
            kept_chunks.push_back(c);
          }
          std::sort(kept_chunks.begin(), kept_chunks.end());
        } else {
          kept_chunks = top_by_score(cand, top_k);
        }
        if (chunk_idx)
          for (int i = 0; i < top_k; ++i)
            chunk_idx[row * top_k + i] = i < (int)kept_chunks.size() ? kept_chunks[i] : -1;

        /* group stage: every group of every kept chunk competes jointly */
        if (group_score)
          for (int g = 0; g < ng; ++g) group_score[row * ng + g] = nan;
        std::vector<std::pair<double, int>> gcand;
        for (int c : kept_chunks)
          for (int t = 0; t < gpc; ++t) {
            const int gam = c * gpc + t;
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += qbar[d] * group_mean[idx4(b, hkv, gam, d, Hkv, ng, D)];
            gcand.push_back({s, gam});
            if (group_score) group_score[row * ng + gam] = s;
          }
        std::vector<int> kept_groups = top_by_score(gcand, top_g);
        if (group_idx)
          for (int i = 0; i < top_g; ++i)
            group_idx[row * top_g + i] = i < (int)kept_groups.size() ? kept_groups[i] : -1;
      }
    }
  return 0;
}

int hgao_route(int B, int Hq, int Hkv, int Sq, int Skv, int D, int C, int G,
               int top_k, int top_g, const double* Q, const double* chunk_mean,
               const double* group_mean, const int32_t* forced_chunk_idx,
               int32_t* chunk_idx, int32_t* group_idx, double* chunk_score,
               double* group_score) {
  return route_impl(B, Hq, Hkv, Sq, Skv, D, C, G, top_k, top_g, Q, false, nullptr, chunk_mean,
                    group_mean, forced_chunk_idx, chunk_idx, group_idx, chunk_score,
                    group_score);
}

/* Strictly causal routing: as hgao_route, but block blk is routed with the
 * mean of the C queries before it (rows (blk-1)C .. blk C - 1 of Q; for
 * blk = 0 the C rows of Qprev, the queries just before the segment, needed
 * only when the segment has history). */
int hgao_route_causal(int B, int Hq, int Hkv, int Sq, int Skv, int D, int C, int G,
                      int top_k, int top_g, const double* Q, const double* Qprev,
                      const double* chunk_mean, const double* group_mean,
                      const int32_t* forced_chunk_idx, int32_t* chunk_idx, int32_t* group_idx,
                      double* chunk_score, double* group_score) {
  return route_impl(B, Hq, Hkv, Sq, Skv, D, C, G, top_k, top_g, Q, true, Qprev, chunk_mean,
                    group_mean, forced_chunk_idx, chunk_idx, group_idx, chunk_score,
                    group_score);
}

/* Exact-token attention (page section "What HGA does differently": only the
 * exact K/V of the kept groups are loaded for the attention itself, and the
 * summaries never serve as keys or values).  The query at absolute position p
 * attends the tokens of its kept groups plus its own chunk up to p.
 * scale <= 0 selects 1/sqrt(D).  lse is the natural-log log-sum-exp of the
 * scaled logits (nullable). */
int hgao_attend_fwd(int B, int Hq, int Hkv, int Sq, int Skv, int D, int C, int G,
                    int top_g, double scale, const double* Q, const double* K,
                    const double* V, const int32_t* group_idx, double* O, double* lse) {
  if (!shape_ok(B, Hq, Hkv, Sq, Skv, D, C, G) || top_g < 0) return 2;
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)D);
  const int r = Hq / Hkv, nblk = Sq / C, q0 = Skv - Sq;
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq) {
      const int hkv = hq / r;
      for (int blk = 0; blk < nblk; ++blk) {
        const long long row = ((long long)b * Hq + hq) * nblk + blk;
        const int cb = q0 / C + blk;
        const int32_t* groups = group_idx + row * top_g;
        if (!groups_valid(groups, top_g, G, C, cb)) return 3;
        for (int i = blk * C; i < blk * C + C; ++i) {
          const int p = q0 + i;
          std::vector<int> keys = key_set(groups, top_g, G, C, cb, p);
          std::vector<double> logit(keys.size());
          double m = -INFINITY;
          for (size_t a = 0; a < keys.size(); ++a) {
            double s = 0.0;
            for (int d = 0; d < D; ++d)
              s += Q[idx4(b, hq, i, d, Hq, Sq, D)] * K[idx4(b, hkv, keys[a], d, Hkv, Skv, D)];
            logit[a] = scale * s;
            m = std::max(m, logit[a]);
          }
          double z = 0.0;
          for (size_t a = 0; a < keys.size(); ++a) z += std::exp(logit[a] - m);
          const double l = m + std::log(z);
          for (int d = 0; d < D; ++d) {
            double o = 0.0;
            for (size_t a = 0; a < keys.size(); ++a)
              o += std::exp(logit[a] - l) * V[idx4(b, hkv, keys[a], d, Hkv, Skv, D)];
            O[idx4(b, hq, i, d, Hq, Sq, D)] = o;
          }
          if (lse) lse[((long long)b * Hq + hq) * Sq + i] = l;
        }
      }
    }
  return 0;
}

/* Backward through the exact-token attention with the routing held fixed (the
 * router has no weights and only scores existing keys, so gradients reach Q, K
 * and V exactly as in dense attention restricted to the attended pairs).
 * The forward is recomputed here from Q, K, V.  dK and dV cover every position
 * and are zero where no query attends. */
int hgao_attend_bwd(int B, int Hq, int Hkv, int Sq, int Skv, int D, int C, int G,
                    int top_g, double scale, const double* Q, const double* K,
                    const double* V, const int32_t* group_idx, const double* dO,
                    double* dQ, double* dK, double* dV) {
  if (!shape_ok(B, Hq, Hkv, Sq, Skv, D, C, G) || top_g < 0) return 2;
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)D);
  const int r = Hq / Hkv, nblk = Sq / C, q0 = Skv - Sq;
  std::memset(dK, 0, sizeof(double) * (size_t)B * Hkv * Skv * D);
  std::memset(dV, 0, sizeof(double) * (size_t)B * Hkv * Skv * D);
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq) {
      const int hkv = hq / r;
      for (int blk = 0; blk < nblk; ++blk) {
        const long long row = ((long long)b * Hq + hq) * nblk + blk;
        const int cb = q0 / C + blk;
        const int32_t* groups = group_idx + row * top_g;
        if (!groups_valid(groups, top_g, G, C, cb)) return 3;
        for (int i = blk * C; i < blk * C + C; ++i) {
          const int p = q0 + i;
          const double* q = Q + idx4(b, hq, i, 0, Hq, Sq, D);
          const double* go = dO + idx4(b, hq, i, 0, Hq, Sq, D);
          std::vector<int> keys = key_set(groups, top_g, G, C, cb, p);
          const size_t n = keys.size();
          /* forward again: logits, softmax, output */
          std::vector<double> logit(n), P(n);
          double m = -INFINITY;
          for (size_t a = 0; a < n; ++a) {
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += q[d] * K[idx4(b, hkv, keys[a], d, Hkv, Skv, D)];
            logit[a] = scale * s;
            m = std::max(m, logit[a]);
          }
          double z = 0.0;
          for (size_t a = 0; a < n; ++a) z += std::exp(logit[a] - m);
          const double l = m + std::log(z);
          for (size_t a = 0; a < n; ++a) P[a] = std::exp(logit[a] - l);
          std::vector<double> o(D, 0.0);
          for (int d = 0; d < D; ++d)
            for (size_t a = 0; a < n; ++a) o[d] += P[a] * V[idx4(b, hkv, keys[a], d, Hkv, Skv, D)];
          /* delta = dO . O */
          double delta = 0.0;
          for (int d = 0; d < D; ++d) delta += go[d] * o[d];
          /* dP, dS and the three gradients */
          double* gq = dQ + idx4(b, hq, i, 0, Hq, Sq, D);
          for (int d = 0; d < D; ++d) gq[d] = 0.0;
          for (size_t a = 0; a < n; ++a) {
            const long long kr = idx4(b, hkv, keys[a], 0, Hkv, Skv, D);
            double dp = 0.0;
            for (int d = 0; d < D; ++d) dp += go[d] * V[kr + d];
            const double ds = P[a] * (dp - delta);
            for (int d = 0; d < D; ++d) {
              gq[d] += scale * ds * K[kr + d];
              dK[kr + d] += scale * ds * q[d];
              dV[kr + d] += P[a] * go[d];
            }
          }
        }
      }
    }
  return 0;
}

/* Decode: one new query per (b, hq), at the last position p = L - 1 of an
 * L-token key/value cache (page section "What HGA does differently", applied
 * to generation: the newest token routes over the resident chunk summaries and
 * attends the exact tokens of its kept groups and of its own chunk).
 * Reading: the routing query of a block that holds a single query is that
 * query; the candidates are the complete chunks strictly before the query's
 * own chunk cp = p / C; the own chunk is attended from its start up to p.
 *   Q [B][Hq][D]; K, V [B][Hkv][L][D]; chunk_mean [B][Hkv][L/C][D];
 *   group_mean [B][Hkv][(L/C)*(C/G)][D]; chunk_idx [B][Hq][top_k];
 *   group_idx [B][Hq][top_g]; O [B][Hq][D]; lse [B][Hq];
 *   chunk_score [B][Hq][L/C], group_score [B][Hq][(L/C)*(C/G)] (NaN where no
 *   candidate), both nullable; forced_chunk_idx [B][Hq][top_k] nullable. */
int hgao_decode(int B, int Hq, int Hkv, int L, int D, int C, int G, int top_k, int top_g,
                double scale, const double* Q, const double* K, const double* V,
                const double* chunk_mean, const double* group_mean,
                const int32_t* forced_chunk_idx, int32_t* chunk_idx, int32_t* group_idx,
                double* O, double* lse, double* chunk_score, double* group_score) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || C <= 0 || G <= 0 || L <= 0) return 2;
  if (Hq % Hkv != 0 || C % G != 0 || top_k < 0 || top_g < 0) return 2;
  if (!all_finite(Q, (long long)B * Hq * D)) return 4;
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)D);
  const int r = Hq / Hkv, gpc = C / G;
  const int nca = L / C, nga = nca * gpc;   /* summary rows present */
  const int p = L - 1, cp = p / C;          /* query position, its own chunk */
  const double nan = std::nan("");
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq) {
      const int hkv = hq / r;
      const long long row = (long long)b * Hq + hq;
      const double* q = Q + row * D;

      /* chunk stage */
      if (chunk_score)
        for (int c = 0; c < nca; ++c) chunk_score[row * nca + c] = nan;
      std::vector<std::pair<double, int>> cand;
      for (int c = 0; c < cp; ++c) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += q[d] * chunk_mean[idx4(b, hkv, c, d, Hkv, nca, D)];
        cand.push_back({s, c});
        if (chunk_score) chunk_score[row * nca + c] = s;
      }
      std::vector<int> kept_chunks;
      if (forced_chunk_idx) {
        for (int i = 0; i < top_k; ++i) {
          const int c = forced_chunk_idx[row * top_k + i];
          if (c < 0) continue;
          if (c >= cp) return 3;
          kept_chunks.push_back(c);
        }
        std::sort(kept_chunks.begin(), kept_chunks.end());
      } else {
        kept_chunks = top_by_score(cand, top_k);
      }
      if (chunk_idx)
        for (int i = 0; i < top_k; ++i)
          chunk_idx[row * top_k + i] = i < (int)kept_chunks.size() ? kept_chunks[i] : -1;

      /* group stage, joint over the kept chunks' groups */
      if (group_score)
        for (int g = 0; g < nga; ++g) group_score[row * nga + g] = nan;
      std::vector<std::pair<double, int>> gcand;
      for (int c : kept_chunks)
        for (int t = 0; t < gpc; ++t) {
          const int gam = c * gpc + t;
          double s = 0.0;
          for (int d = 0; d < D; ++d) s += q[d] * group_mean[idx4(b, hkv, gam, d, Hkv, nga, D)];
          gcand.push_back({s, gam});
          if (group_score) group_score[row * nga + gam] = s;
        }
      std::vector<int> kept_groups = top_by_score(gcand, top_g);
      std::vector<int32_t> groups(top_g > 0 ? top_g : 1, -1);
      for (int i = 0; i < top_g; ++i)
        groups[i] = i < (int)kept_groups.size() ? kept_groups[i] : -1;
      if (group_idx)
        for (int i = 0; i < top_g; ++i) group_idx[row * top_g + i] = groups[i];

      /* exact-token attention of the query over its key set */
      std::vector<int> keys = key_set(groups.data(), top_g, G, C, cp, p);
      std::vector<double> logit(keys.size());
      double m = -INFINITY;
      for (size_t a = 0; a < keys.size(); ++a) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += q[d] * K[idx4(b, hkv, keys[a], d, Hkv, L, D)];
        logit[a] = scale * s;
        m = std::max(m, logit[a]);
      }
      double z = 0.0;
      for (size_t a = 0; a < keys.size(); ++a) z += std::exp(logit[a] - m);
      const double l = m + std::log(z);
      for (int d = 0; d < D; ++d) {
        double o = 0.0;
        for (size_t a = 0; a < keys.size(); ++a)
          o += std::exp(logit[a] - l) * V[idx4(b, hkv, keys[a], d, Hkv, L, D)];
        O[row * D + d] = o;
      }
      if (lse) lse[row] = l;
    }
  return 0;
}

/* Number of attended (query, key) pairs summed over every query of every head:
 * the algorithmic work count of the attention (each kept group contributes G
 * keys to all C queries of its block, the own chunk C(C+1)/2 causal pairs). */
long long hgao_attended_pairs(int B, int Hq, int Sq, int C, int G, int top_g,
                              const int32_t* group_idx) {
  const int nblk = Sq / C;
  long long pairs = 0;
  for (long long row = 0; row < (long long)B * Hq * nblk; ++row) {
    int kept = 0;
    for (int i = 0; i < top_g; ++i)
      if (group_idx[row * top_g + i] >= 0) ++kept;
    pairs += (long long)C * G * kept + (long long)C * (C + 1) / 2;
  }
  return pairs;
}

}  /* extern "C" */

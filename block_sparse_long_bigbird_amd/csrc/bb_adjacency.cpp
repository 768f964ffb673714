// Host-side random-block table for BigBird block-sparse attention.
//
// Source: page "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
// section "随机块掩码是如何生成的": for every head, one row per middle block; each
// row takes num_rand_blocks ids from the middle block ids (first and last
// block removed) with the row's own window removed, so random blocks never
// overlap the band.  The reference draws them with numpy's permutation at
// layer-build time; its bit stream cannot be reproduced from the page, so this
// builder defines its own: the first r entries of a uniformly random
// permutation of the candidates, i.e. a uniform r-subset, stored sorted.
//
// Generators (published definitions):
//   SplitMix64 -- G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
//                 pseudorandom number generators", OOPSLA 2014.
//   bounded draws -- D. Lemire, "Fast random integer generation in an
//                 interval", ACM TOMACS 2019 (multiply-shift with rejection).
//
// Plain C++17, no HIP: this translation unit also builds with g++ alone.

#include <algorithm>
#include <cstdint>
#include <vector>

#include "bb_attn.h"

namespace {

struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

// Uniform integer in [0, range), range >= 1 (Lemire 2019).
uint64_t bounded(SplitMix64& g, uint64_t range) {
  unsigned __int128 m = static_cast<unsigned __int128>(g.next()) * range;
  uint64_t low = static_cast<uint64_t>(m);
  if (low < range) {
    const uint64_t threshold = (0 - range) % range;
    while (low < threshold) {
      m = static_cast<unsigned __int128>(g.next()) * range;
      low = static_cast<uint64_t>(m);
    }
  }
  return static_cast<uint64_t>(m >> 64);
}

// Stream of head h: the seed mixed with the head index through one SplitMix64
// output, so neighbouring heads start far apart.
SplitMix64 head_stream(uint64_t seed, int h) {
  SplitMix64 mix{seed ^ (0xD1B54A32D192ED03ull * static_cast<uint64_t>(h + 1))};
  return SplitMix64{mix.next()};
}

int check_sizes(int H, int L, int block, int r, int* nb_out) {
  if (H < 0 || L <= 0 || block <= 0 || r < 0) return BB_ERR_SHAPE;
  if (L % block != 0) return BB_ERR_SHAPE;
  const int nb = L / block;
  if (nb < 3) return BB_ERR_SHAPE;
  const int r_max = nb - 5 > 0 ? nb - 5 : 0;  // interior rows have nb-5 candidates
  if (r > r_max) return BB_ERR_SHAPE;
  *nb_out = nb;
  return BB_OK;
}

// The table with random candidates limited to blocks j <= jmax (jmax >= nb-2:
// no limit).  Every row must keep at least r candidates.
int build_table(uint64_t seed, int H, int nb, int r, int jmax, int32_t* rand_idx) {
  std::vector<int32_t> cand;
  cand.reserve(nb);
  const int hi = jmax < nb - 2 ? jmax : nb - 2;
  for (int i = 1; i <= nb - 2; ++i) {
    int n = 0;
    for (int j = 1; j <= hi; ++j) n += (j < i - 1 || j > i + 1) ? 1 : 0;
    if (n < r) return BB_ERR_SHAPE;
  }
  for (int h = 0; h < H; ++h) {
    SplitMix64 g = head_stream(seed, h);
    for (int i = 1; i <= nb - 2; ++i) {
      cand.clear();
      for (int j = 1; j <= hi; ++j)
        if (j < i - 1 || j > i + 1) cand.push_back(j);
      const int n = static_cast<int>(cand.size());
      for (int t = 0; t < r; ++t) {  // partial Fisher-Yates: first r of a uniform permutation
        const int pick = t + static_cast<int>(bounded(g, static_cast<uint64_t>(n - t)));
        std::swap(cand[t], cand[pick]);
      }
      std::sort(cand.begin(), cand.begin() + r);
      int32_t* row = rand_idx + (static_cast<size_t>(h) * (nb - 2) + (i - 1)) * r;
      std::copy(cand.begin(), cand.begin() + r, row);
    }
  }
  return BB_OK;
}

}  // namespace

extern "C" int bb_rand_idx_build(uint64_t seed, int H, int L, int block, int r, int32_t* rand_idx) {
  int nb = 0;
  const int st = check_sizes(H, L, block, r, &nb);
  if (st != BB_OK) return st;
  if (H == 0 || r == 0) return BB_OK;
  if (rand_idx == nullptr) return BB_ERR_NULL;
  return build_table(seed, H, nb, r, nb - 2, rand_idx);
}

extern "C" int bb_rand_idx_build_capped(uint64_t seed, int H, int L, int block, int r, int last_idx,
                                        int32_t* rand_idx) {
  int nb = 0;
  const int st = check_sizes(H, L, block, r, &nb);
  if (st != BB_OK) return st;
  if (last_idx <= 0) return bb_rand_idx_build(seed, H, L, block, r, rand_idx);
  // a block counts when it lies wholly before token last_idx
  const int jmax = last_idx / block - 1;
  if (H == 0 || r == 0) return BB_OK;
  if (rand_idx == nullptr) return BB_ERR_NULL;
  return build_table(seed, H, nb, r, jmax, rand_idx);
}

extern "C" int bb_rand_idx_check(const int32_t* rand_idx, int H, int L, int block, int r) {
  int nb = 0;
  const int st = check_sizes(H, L, block, r, &nb);
  if (st != BB_OK) return st;
  if (H == 0 || r == 0) return BB_OK;
  if (rand_idx == nullptr) return BB_ERR_NULL;
  for (int h = 0; h < H; ++h) {
    for (int i = 1; i <= nb - 2; ++i) {
      const int32_t* row = rand_idx + (static_cast<size_t>(h) * (nb - 2) + (i - 1)) * r;
      for (int t = 0; t < r; ++t) {
        const int32_t e = row[t];
        if (e < 1 || e > nb - 2) return BB_ERR_RAND_IDX;
        if (e >= i - 1 && e <= i + 1) return BB_ERR_RAND_IDX;
        for (int u = 0; u < t; ++u)
          if (row[u] == e) return BB_ERR_RAND_IDX;
      }
    }
  }
  return BB_OK;
}

extern "C" int bb_rand_idx_invert(const int32_t* rand_idx, int H, int L, int block, int r, int32_t* inv_off,
                                  int32_t* inv_rows) {
  const int st = bb_rand_idx_check(rand_idx, H, L, block, r);
  if (st != BB_OK) return st;
  const int nb = L / block;
  if (H == 0) return BB_OK;
  if (inv_off == nullptr || (r > 0 && inv_rows == nullptr)) return BB_ERR_NULL;
  const size_t per_head = static_cast<size_t>(nb - 2) * r;
  for (int h = 0; h < H; ++h) {
    int32_t* off = inv_off + static_cast<size_t>(h) * (nb + 1);
    for (int j = 0; j <= nb; ++j) off[j] = 0;
    // counts per key block, then exclusive prefix sums (absolute offsets)
    for (size_t e = 0; e < per_head; ++e) ++off[rand_idx[h * per_head + e] + 1];
    off[0] = static_cast<int32_t>(h * per_head);
    for (int j = 1; j <= nb; ++j) off[j] += off[j - 1];
    // fill in increasing row order: rows come out ascending within each key block
    std::vector<int32_t> cursor(off, off + nb);
    for (int i = 1; i <= nb - 2; ++i)
      for (int t = 0; t < r; ++t) {
        const int j = rand_idx[h * per_head + static_cast<size_t>(i - 1) * r + t];
        inv_rows[cursor[j]++] = i;
      }
  }
  return BB_OK;
}

// msa_select.h -- step 3 on one wave: top-k block selection with the latest
// block kept (vLLM M3.1 post, "MiniMax 稀疏注意力的工作原理"; "MiniMax goes
// sparse", section 1 Step 1, TopK per layer and GQA group).  Used by the
// selection kernel and by the fused selection + attention kernel.
//
// Each candidate block becomes a 64-bit key: the order-preserving image of
// its FP32 score in the high word (-0 folded onto +0, NaN below every
// number) and 0xFFFFFFFF - j in the low word, so the larger key is the better
// block and equal scores go to the lower block index.  topk-1 rounds of a
// wave-wide argmax pick the best blocks other than the latest.
//
// Each lane keeps its candidates' keys in registers (KMAX per lane, blocks
// lane, lane+64, ...; KMAX = 0 reads them from memory when needed, for very
// long contexts) and a sorted list of its own best 3.  A round takes the
// wave-wide max of the list heads -- one 32-bit DPP max of the score words
// and a ballot; a second reduction of the index words runs only when several
// heads carry the same score -- and the winning lane pops its head.  A lane
// whose list runs dry refills it from its keys below the key it just gave up
// (keys are distinct, so "below the last winner" is exactly "not yet
// selected").
#pragma once

#include "msa_device.h"

namespace msa {

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (f == f) ? k : 0u;  // NaN ranks below -inf
}

template <bool kTok>
__device__ __forceinline__ float block_score(const float* __restrict__ row, int j, int pos_lim) {
  if (!kTok) return row[j];
  float m = -__builtin_inff();
  const int hi = min(kPage - 1, pos_lim - j * kPage);
  for (int t = 0; t <= hi; ++t) m = fmaxf(m, row[j * kPage + t]);
  return m;
}

// Insert key k into a descending top-3 list (0 = empty slot).
__device__ __forceinline__ void top3_insert(uint64_t k, uint64_t& t0, uint64_t& t1, uint64_t& t2) {
  const bool g0 = k > t0, g1 = k > t1, g2 = k > t2;
  t2 = g1 ? t1 : (g2 ? k : t2);
  t1 = g0 ? t0 : (g1 ? k : t1);
  t0 = g0 ? k : t0;
}

// Scores of candidate blocks j = lane + 64 i (i < KMAX) of a block-score row
// with `cap` entries, loaded before the row length is known: the index is
// clamped into the row and candidates past the latest block are masked by the
// selection.  Every load is unconditional, so they issue back to back.
template <int KMAX>
__device__ __forceinline__ void load_row_scores(const float* __restrict__ row, int cap, int lane,
                                                float (&sc)[KMAX > 0 ? KMAX : 1]) {
#pragma unroll
  for (int i = 0; i < KMAX; ++i) sc[i] = row[min(lane + 64 * i, cap - 1)];
}

// Selection of one (request, row, group) by one whole wave, n = number of
// blocks the row sees.  With KMAX > 0, sc holds the scores of this lane's
// candidates (blocks lane + 64 i; entries for j >= n - 1 are ignored); with
// KMAX == 0, score_of(j) reads them on demand.  Calls emit(rank, id) once for
// each selected block (rank = position in ascending order) from the lane that
// holds it, and returns the count.
template <int KMAX, typename ScoreOf, typename Emit>
__device__ __forceinline__ int select_core(const float (&sc)[KMAX > 0 ? KMAX : 1], ScoreOf score_of, int n,
                                           int topk, int lane, Emit emit) {
  if (n <= topk) {
    if (lane < n) emit(lane, lane);
    return n;
  }
  const int latest = n - 1;
  auto key_of = [&](int j, float s) {
    return ((uint64_t)order_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
  };
  uint64_t keys[KMAX > 0 ? KMAX : 1];
  uint64_t t0 = 0, t1 = 0, t2 = 0;
  if (KMAX > 0) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const int j = lane + 64 * i;
      keys[i] = j < latest ? key_of(j, sc[i]) : 0ull;
      top3_insert(keys[i], t0, t1, t2);
    }
  } else {
    for (int j = lane; j < latest; j += 64) top3_insert(key_of(j, score_of(j)), t0, t1, t2);
  }
  int mine = -1;  // the block this lane ends up holding in the output set
  for (int k = 0; k < topk - 1; ++k) {
    const uint32_t hi = (uint32_t)(t0 >> 32);
    const uint32_t H = wave_umax(hi);
    const uint64_t tied = __ballot(hi == H);
    int wl;
    if (__popcll(tied) == 1) {
      wl = __ffsll((unsigned long long)tied) - 1;
    } else {  // equal scores: the lower block index (larger low word) wins
      const uint32_t Lo = wave_umax(hi == H ? (uint32_t)t0 : 0u);
      wl = (int)((0xFFFFFFFFu - Lo) & 63u);
    }
    const uint64_t W = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(t0 >> 32), wl) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)t0, wl);
    if (lane == k) mine = (int)(0xFFFFFFFFu - (uint32_t)W);
    if (lane == wl) {
      t0 = t1;
      t1 = t2;
      t2 = 0;
      if (t0 == 0) {  // list ran dry: refill from this lane's keys below W
        if (KMAX > 0) {
#pragma unroll
          for (int i = 0; i < KMAX; ++i)
            if (keys[i] < W) top3_insert(keys[i], t0, t1, t2);
        } else {
          for (int j = lane; j < latest; j += 64) {
            const uint64_t kk = key_of(j, score_of(j));
            if (kk < W) top3_insert(kk, t0, t1, t2);
          }
        }
      }
    }
  }
  if (lane == topk - 1) mine = latest;
  // rank of each held id among the held ids (ids are distinct)
  int rank = 0;
  for (int i = 0; i < topk; ++i) {
    const int other = __builtin_amdgcn_readlane(mine, i);
    rank += (lane < topk && other < mine) ? 1 : 0;
  }
  if (lane < topk) emit(rank, mine);
  return topk;
}

constexpr float kNoScores[1] = {0.f};  // select_core<0> reads its scores through score_of

// Per-wave LDS scratch of select_fast.
constexpr int kSelCand = 512;  // candidate capacity (beyond it: the round-based selection)
struct SelectScratch {
  uint64_t cand[kSelCand + 64];  // candidates, then one discard slot per lane
  int pick[64];                  // picked block ids by key rank
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t lanes_below_mask(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Number of lanes in a ballot, as a 32-bit count (kept on the scalar unit).
__device__ __forceinline__ int ballot_count(uint64_t b) {
  return __builtin_popcount((uint32_t)b) + __builtin_popcount((uint32_t)(b >> 32));
}

// The k-th largest (k >= 1) of the wave's 32-bit lane values, all lanes
// active: bitwise from the top, the largest c with at least k lanes >= c (one
// ballot count per bit).
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, int k) {
  uint32_t th = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = th | (1u << bit);
    if (ballot_count(__ballot(v >= c)) >= k) th = c;
  }
  return th;
}

// The same selection as select_core with no serial rounds.  Candidate block
// j (< latest) gets the 32-bit score key ck = order_key + 1 (absent blocks 0)
// and the 64-bit key (ck, 0xFFFFFFFF - j), ordered as select_core's keys.
// With need = topk - 1 blocks to pick besides the latest:
//  1. each lane takes the max of its candidates' score keys (its "head");
//  2. T = the need-th largest head (wave_kth_largest; at least need lanes
//     hold a candidate, so T >= 1);
//  3. the need largest keys all have score keys >= T (the need lanes with
//     heads >= T hold need keys at least that large), so the keys with
//     ck >= T -- compacted into LDS -- include them; with distinct scores
//     they come only from those need lanes;
//  4. a candidate's rank among the candidates is its rank among all keys: the
//     need best are picked, and each one's place in ascending block order is
//     the number of picked ids below it.
// Beyond kSelCand candidates (many equal scores) it runs select_core
// instead, reading the scores again through score_of (so that the register
// copies need not stay live).  S: this wave's scratch.
template <int KMAX, typename ScoreOf, typename Emit>
__device__ __forceinline__ int select_fast(const float (&sc)[KMAX > 0 ? KMAX : 1], ScoreOf score_of, int n, int topk,
                                           int lane, SelectScratch* S, Emit emit) {
  if (n <= topk) {
    if (lane < n) emit(lane, lane);
    return n;
  }
  const int latest = n - 1;
  const int need = topk - 1;
  if (need == 0) {
    if (lane == 0) emit(0, latest);
    return 1;
  }
  // score key of block j (a candidate, j < latest), or 0; branch-free
  auto ck_of = [&](int j, float s) { return (order_key(s) + 1u) & (0u - (uint32_t)(j < latest)); };
  auto key64 = [](uint32_t ck, int j) { return ((uint64_t)ck << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j); };
  uint32_t ck[KMAX > 0 ? KMAX : 1];
  uint32_t head = 0;
  if (KMAX > 0) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) ck[i] = ck_of(lane + 64 * i, sc[i]);
    // pairwise tree: independent maxima issue back to back
    uint32_t t[KMAX > 0 ? KMAX : 1];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) t[i] = ck[i];
#pragma unroll
    for (int w = 1; w < KMAX; w *= 2)
#pragma unroll
      for (int i = 0; i + w < KMAX; i += 2 * w) t[i] = max(t[i], t[i + w]);
    head = t[0];
  } else {
    for (int j = lane; j < latest; j += 64) head = max(head, ck_of(j, score_of(j)));
  }
  const uint32_t T = wave_kth_largest(head, need);
  const uint64_t below = lanes_below_mask(lane);
  int C = 0;
  if (KMAX > 0) {
    // each lane's candidates go to consecutive slots after those of the lanes
    // below it (an exclusive count summed from ballots of the count's bits);
    // other keys go to the lane's discard slot, so every store is unconditional
    int mine = 0;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) mine += ck[i] >= T ? 1 : 0;
    int off = 0;
#pragma unroll
    for (int bit = 0; (1 << bit) <= KMAX; ++bit) {
      const uint64_t bal = __ballot((mine >> bit) & 1);
      off += ballot_count(bal & below) << bit;
      C += ballot_count(bal) << bit;
    }
    if (C > kSelCand) return select_core<0>(kNoScores, score_of, n, topk, lane, emit);
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const bool c = ck[i] >= T;
      S->cand[c ? off : kSelCand + lane] = key64(ck[i], lane + 64 * i);
      off += c ? 1 : 0;
    }
  } else {
    for (int base = 0; base < latest; base += 64) {
      const int j = base + lane;
      const uint32_t k = ck_of(j, score_of(min(j, latest - 1)));
      const bool c = k >= T;
      const uint64_t bal = __ballot(c);
      const int off = C + ballot_count(bal & below);
      if (c && off < kSelCand) S->cand[off] = key64(k, j);
      C += ballot_count(bal);
    }
    if (C > kSelCand) return select_core<0>(kNoScores, score_of, n, topk, lane, emit);
  }
  wave_lds_sync();
  for (int base = 0; base < C; base += 64) {
    const int c = base + lane;
    const uint64_t mine = c < C ? S->cand[c] : 0ull;
    int r = 0;
    for (int m = 0; m < C; ++m) r += S->cand[m] > mine ? 1 : 0;
    if (c < C && r < need) S->pick[r] = (int)(0xFFFFFFFFu - (uint32_t)mine);
  }
  wave_lds_sync();
  if (lane < need) {
    const int id = S->pick[lane];
    int pos = 0;
    for (int m = 0; m < need; ++m) pos += S->pick[m] < id ? 1 : 0;
    emit(pos, id);
  }
  if (lane == 0) emit(need, latest);
  return topk;
}

// Selection from a score row in memory (block scores, or token scores when
// kTok: a block then scores the max of its visible tokens); p is the row's
// position.
template <bool kTok, int KMAX, typename Emit>
__device__ __forceinline__ int select_row(const float* __restrict__ row, int n, int p, int topk, int lane,
                                          Emit emit) {
  float sc[KMAX > 0 ? KMAX : 1];
  const int last = max(n - 2, 0);  // highest candidate (the latest block is kept apart)
#pragma unroll
  for (int i = 0; i < KMAX; ++i) sc[i] = block_score<kTok>(row, min(lane + 64 * i, last), p);
  return select_core<KMAX>(sc, [&](int j) { return block_score<kTok>(row, j, p); }, n, topk, lane, emit);
}

// Register capacity (candidates per lane) for a block-table width.
__host__ __device__ constexpr int select_kmax(int max_pages) {
  return max_pages <= 64 * 8 ? 8 : (max_pages <= 64 * 24 ? 24 : (max_pages <= 64 * 48 ? 48 : 0));
}

}  // namespace msa

// The seeded Gumbel draw that ends the transform program (xorl issue #71,
// section 3: temperature -> stable token-id top-k -> inclusive top-p -> min-p
// -> seeded Gumbel).  The pages name the stage without defining its
// generator; the draw here:
//   r_v   = word (v mod 4) of Philox4x32-10(counter = (v div 4, row, offset
//           low, offset high), key = (seed low, seed high)) - the generator of
//           Salmon, Moraes, Dror and Shaw ("Parallel random numbers: as easy as
//           1, 2, 3", SC 2011), written from its definition;
//   u_v   = (r_v + 1/2) 2^-32, strictly inside (0, 1);
//   draw  = the support token with the largest (x_v - x_max) / tau - ln(-ln u_v)
//           in fp64, the lower id on equal scores.
// The support is the transforms' descriptor: every token with x above the
// threshold logit, and the first threshold_ties tokens (by id) equal to it.
//
// One workgroup per row streams the row once, two chunks ahead of the one it
// scores.  Every token at or above the threshold gets an fp32 score with a
// bound on its error (its Philox block computed once per 4 tokens); each
// thread keeps its best by the upper end of that interval (its id only, a few
// selects per token), so the fp64 score - the decision - is taken only for
// the few tokens that can still be the best, without divergent fp64 work in
// the loop.  Tokens equal to the threshold are tracked apart.  When the row
// holds more threshold-equal tokens than the support takes, a second pass
// ranks them by id and keeps the best of the first threshold_ties: rows of
// up to 155,648 tokens rank them from per-chunk tie counts kept in LDS during
// the first pass (one scan), longer rows by a block scan per round of chunks.
#include "common.h"
#include "launch.h"

namespace vs {

namespace {

// 512 threads and 78 KiB of LDS: two rows per CU, so one row's reductions
// overlap the other's stream
constexpr int kSampleThreads = 512;
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct Ctr {
  uint32_t c0, c1, c2, c3;
};

// Ten Philox rounds: words 0 and 2 are multiplied into 64-bit products, the
// high halves are mixed with words 1 and 3 and the key, the key grows by the
// Weyl increments after every round.
__device__ __forceinline__ Ctr philox4x32_10(Ctr c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = uint64_t(kPhiloxM0) * c.c0;
    const uint64_t p1 = uint64_t(kPhiloxM1) * c.c2;
    Ctr n;  // (three-way XORs as one gfx950 three-input bit operation each: truth table 0x96)
    n.c0 = __builtin_amdgcn_bitop3_b32(uint32_t(p1 >> 32), c.c1, k0, 0x96);
    n.c1 = uint32_t(p1);
    n.c2 = __builtin_amdgcn_bitop3_b32(uint32_t(p0 >> 32), c.c3, k1, 0x96);
    n.c3 = uint32_t(p0);
    c = n;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return c;
}

__device__ __forceinline__ uint32_t ctr_word(const Ctr& c, int j) {
  return j == 0 ? c.c0 : j == 1 ? c.c1 : j == 2 ? c.c2 : c.c3;
}

struct Best {
  double s;
  int64_t id;
};

__device__ __forceinline__ bool better(const Best& a, const Best& b) { return a.s > b.s || (a.s == b.s && a.id < b.id); }

__device__ __forceinline__ Best wave_best(Best b) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Best o;
    o.s = __shfl_xor(b.s, off, 64);
    o.id = __shfl_xor(b.id, off, 64);
    if (better(o, b)) b = o;
  }
  return b;
}

// Rows of up to kLdsChunks 8-token chunks keep one tie count per chunk in LDS
// (then an exclusive scan in place): V <= 155,648.
constexpr int kLdsChunks = 19456;

struct SampleSmem {
  double best_s[kSampleThreads / 64];
  int64_t best_id[kSampleThreads / 64];
  uint32_t wcount[2][kSampleThreads / 64];
  uint32_t chunk_ties[kLdsChunks];
};

// The workgroup's best of every thread's candidate, in every thread.
__device__ __forceinline__ Best block_best(Best b, SampleSmem& sm) {
  constexpr int NW = kSampleThreads / 64;
  b = wave_best(b);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sm.best_s[w] = b.s;
    sm.best_id[w] = b.id;
  }
  __syncthreads();
  Best r{sm.best_s[0], sm.best_id[0]};
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    const Best o{sm.best_s[i], sm.best_id[i]};
    if (better(o, r)) r = o;
  }
  return r;
}

// Exclusive prefix of c over the workgroup's threads and the total (every
// thread); `buf` alternates between two LDS slots so consecutive calls need
// one barrier each.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t c, uint32_t& total, SampleSmem& sm, int buf) {
  constexpr int NW = kSampleThreads / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) sm.wcount[buf][w] = inc;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t t = sm.wcount[buf][i];
    before += i < w ? t : 0u;
    total += t;
  }
  return before + inc - c;
}

// Chunk q of a row: tokens 8q .. 8q+7; past V a NaN, which compares false with
// any threshold (a -inf threshold included).
__device__ __forceinline__ void load_chunk(const uint16_t* rowp, bool vec, int64_t q, int V, float* x) {
  const int64_t v0 = 8 * q;
  if (vec && v0 + 8 <= V) {
    const uint4 w = *reinterpret_cast<const uint4*>(rowp + v0);
    x[0] = bf16_lo(w.x);
    x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y);
    x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z);
    x[5] = bf16_hi(w.z);
    x[6] = bf16_lo(w.w);
    x[7] = bf16_hi(w.w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = v0 + i < V ? bf16_to_f32(rowp[v0 + i]) : __builtin_nanf("");
  }
}

struct DrawArgs {
  int64_t row;
  double tau, xmax;
  float xmaxf, inv_tau;
  uint32_t k0, k1, off_lo, off_hi;
};

// The Gumbel score of token v from its 32-bit number r, in fp64: the decision.
__device__ __forceinline__ double gumbel_score(float x, uint32_t r, const DrawArgs& d) {
  const double u = (double(r) + 0.5) * 0x1p-32;
  const double g = -log(-log(u));
  return (double(x) - d.xmax) / d.tau + g;
}

// The same score in fp32, and a bound on its distance from the fp64 one.
// -ln u: from u rounded to 24 bits, which moves -ln u by at most 2^-14 of its
// value while u < 1 - 2^-10; above that, from the series eps + eps^2/2 +
// eps^3/3 in eps = 1 - u, exact in fp32 there (truncation below 2^-30
// relative).  With two fp32 logarithms and the product, the score is off by
// less than 2^-21 |dz| + 1e-4; the bound returned, 2^-18 |dz| + 1e-3, has a
// wide margin.
__device__ __forceinline__ float score32(float x, uint32_t r, const DrawArgs& d, float& err) {
  float e;
  if (r >= 0xFFC00000u) {
    const float eps = (float(0xFFFFFFFFu - r) + 0.5f) * 0x1p-32f;
    e = eps * (1.0f + eps * (0.5f + eps * (1.0f / 3.0f)));
  } else {
    e = -kLn2 * log2_hw((float(r) + 0.5f) * 0x1p-32f);
  }
  const float g = -kLn2 * log2_hw(e);
  const float dz = (x - d.xmaxf) * d.inv_tau;
  err = 0x1p-18f * fabsf(dz) + 1e-3f;
  return dz + g;
}

// A thread's best token of one category by the upper end of its fp32 score
// interval (the lower id on equal ends), the largest upper end of every other
// token, and the largest lower end of all.  The true best token of a category
// has its upper end at or above every lower end, so it is a kept token whose
// upper end reaches the workgroup's largest lower end - unless some other
// token's upper end reaches it too, which the caller detects from b2 and then
// rescans.  Only the id is kept: the token's logit and number are recomputed
// for the one or two tokens the decision needs.
struct Top1 {
  float hi1, b2, max_lo;
  int32_t id1;
};
__device__ __forceinline__ Top1 top1_empty(int V) {
  const float ni = -__builtin_inff();
  return Top1{ni, ni, ni, V};
}
__device__ __forceinline__ void top1_add(Top1& t, float s, float err, int32_t id) {
  const float hi = s + err;
  t.max_lo = fmaxf(t.max_lo, s - err);
  const bool take = hi > t.hi1 || (hi == t.hi1 && id < t.id1);
  t.b2 = fmaxf(t.b2, take ? t.hi1 : hi);
  t.hi1 = take ? hi : t.hi1;
  t.id1 = take ? id : t.id1;
}

__device__ __forceinline__ float block_max_f(float v, SampleSmem& sm) {
  constexpr int NW = kSampleThreads / 64;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.best_s[threadIdx.x >> 6] = double(v);
  __syncthreads();
  float r = float(sm.best_s[0]);
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, float(sm.best_s[i]));
  return r;
}

__global__ __launch_bounds__(kSampleThreads) void sample_kernel(
    const uint16_t* __restrict__ logits, int64_t ld, int V, const float* __restrict__ temp, float temp_scalar,
    const uint8_t* __restrict__ status, const float* __restrict__ threshold_logit,
    const int32_t* __restrict__ threshold_ties, const float* __restrict__ row_max, uint64_t seed, uint64_t offset,
    int64_t* __restrict__ sampled, uint8_t* __restrict__ out_status, int64_t row0, const int32_t* __restrict__ order,
    const int64_t* __restrict__ ids, int cap, const int32_t* __restrict__ support_len) {
  __shared__ SampleSmem sm;
  // local row (taken in the order `order` gives, when given); row0 + row is
  // the generator's row word, so the order changes no draw
  const int64_t row = order ? int64_t(order[blockIdx.x]) : int64_t(blockIdx.x);
  const int tid = threadIdx.x;
  if (tid == 0 && out_status) out_status[row] = status[row] & kRowBad;
  if (status[row] & kRowBad) {
    if (tid == 0) sampled[row] = -1;
    return;
  }
  DrawArgs d;
  d.row = row0 + row;
  d.tau = double(temp ? temp[row] : temp_scalar);
  d.xmax = double(row_max[row]);
  d.xmaxf = row_max[row];
  d.inv_tau = 1.0f / float(d.tau);
  d.k0 = uint32_t(seed);
  d.k1 = uint32_t(seed >> 32);
  d.off_lo = uint32_t(offset);
  d.off_hi = uint32_t(offset >> 32);
  const uint16_t* rowp = logits + row * ld;
  const auto block_ctr = [&](int64_t q, int b) {
    return philox4x32_10(Ctr{uint32_t(2 * q + b), uint32_t(d.row), d.off_lo, d.off_hi}, d.k0, d.k1);
  };
  // A support of at most cap (<= 64) tokens whose dense ids the transforms
  // wrote: one lane per id scores it in fp64 (the decision itself), no row pass.
  if (ids) {
    const int32_t L = support_len[row];
    if (L >= 1 && L <= cap) {
      if (tid >= 64) return;
      Best b{-__builtin_inf(), int64_t(V)};
      if (tid < L) {
        const int64_t id = ids[row * cap + tid];
        const float x = bf16_to_f32(rowp[id]);
        if (x != -__builtin_inff()) {
          const Ctr r = block_ctr(id >> 3, int((id >> 2) & 1));
          b = Best{gumbel_score(x, ctr_word(r, int(id & 3)), d), id};
        }
      }
      b = wave_best(b);
      if (tid == 0) sampled[row] = b.id;
      return;
    }
  }
  const float thr = threshold_logit[row];
  const uint32_t ties = uint32_t(threshold_ties[row]);
  const bool vec = (reinterpret_cast<uintptr_t>(rowp) & 15) == 0;
  const int64_t nchunk = (int64_t(V) + 7) / 8;
  const bool lds_ranks = nchunk <= kLdsChunks;

  // Every token above the threshold (f_gt) and every token equal to it
  // (f_eq, with its count written to LDS when lds_ranks): one pass over the row.
  // The raw bf16 bits of chunk q (NaN past V, which no threshold admits).
  auto load_raw = [&](int64_t q) -> uint4 {
    if (vec && 8 * q + 8 <= V) return *reinterpret_cast<const uint4*>(rowp + 8 * q);
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = 8 * q + i < V ? uint32_t(rowp[8 * q + i]) : 0x7FC0u;
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  };
  // The row pass.  An aligned row's first 4 * floor(nfull / (4 NT)) * NT whole
  // 16-byte chunks go through a ring of four loads per thread in fixed slots
  // (a slot is copied, refilled with the chunk four ahead, then scored; the
  // refills past the ring's last chunk re-read it, unused), so each wait is
  // for the oldest load alone and no register moves under a load in flight;
  // the thread's remaining chunks (and every chunk of an unaligned row) are
  // loaded one by one.  A thread's chunks are scored in ascending order.
  auto each_token = [&](bool count_ties, auto f_gt, auto f_eq) {
    uint32_t n_eq = 0;
    constexpr int64_t NT = kSampleThreads;
    auto chunk = [&](int64_t q, const uint4& w) {
      float x[8];
      x[0] = bf16_lo(w.x);
      x[1] = bf16_hi(w.x);
      x[2] = bf16_lo(w.y);
      x[3] = bf16_hi(w.y);
      x[4] = bf16_lo(w.z);
      x[5] = bf16_hi(w.z);
      x[6] = bf16_lo(w.w);
      x[7] = bf16_hi(w.w);
      if (count_ties && lds_ranks) {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) c += x[i] == thr ? 1u : 0u;
        sm.chunk_ties[q] = c;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        bool any = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) any |= x[4 * b + i] >= thr;
        if (!any) continue;
        const Ctr r = block_ctr(q, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xv = x[4 * b + i];
          if (!(xv >= thr)) continue;
          const int64_t id = 8 * q + 4 * b + i;
          if (xv == thr) {
            ++n_eq;
            f_eq(xv, ctr_word(r, i), id);
          } else {
            f_gt(xv, ctr_word(r, i), id);
          }
        }
      }
    };
    const int64_t n4 = vec ? int64_t(V) / 8 / (4 * NT) * 4 : 0;  // ring chunks per thread (uniform)
    if (n4 > 0) {
      const uint4* pv = reinterpret_cast<const uint4*>(rowp) + tid;
      // the thread's k-th chunk, a streaming (non-temporal) load: the row is
      // read once here
      auto ld = [&](int64_t k) { return stream_load(pv + (k < n4 ? k : n4 - 1) * NT); };
      uint4 b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) b[u] = ld(u);
      for (int64_t i = 0; i < n4; i += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 w = b[u];
          b[u] = ld(i + u + 4);
          chunk(tid + (i + u) * NT, w);
        }
      }
    }
    for (int64_t q = n4 * NT + tid; q < nchunk; q += NT) chunk(q, load_raw(q));
    return n_eq;
  };
  // The first `ties` threshold-equal tokens by id (f), when the row holds
  // more: ranked from the LDS chunk counts of the first pass (`ranked` tells
  // that the in-place scan has run), or by a block scan per round of chunks.
  // Every thread calls it (barriers inside).
  bool ranked = false;
  auto each_ranked_tie = [&](auto f) {
    if (lds_ranks) {
      if (!ranked) {
        const int64_t seg = (nchunk + kSampleThreads - 1) / kSampleThreads;
        const int64_t s0 = tid * seg, s1 = s0 + seg < nchunk ? s0 + seg : nchunk;
        uint32_t run = 0;
        for (int64_t q = s0; q < s1; ++q) run += sm.chunk_ties[q];
        uint32_t total;
        uint32_t acc = block_excl_scan(run, total, sm, 1);
        for (int64_t q = s0; q < s1; ++q) {
          const uint32_t c = sm.chunk_ties[q];
          sm.chunk_ties[q] = acc;
          acc += c;
        }
        if (tid == 0) sm.wcount[0][0] = total;  // (wcount[0] is free again: the last scan used slot 1)
        __syncthreads();
        ranked = true;
      }
      const uint32_t total = sm.wcount[0][0];
      for (int64_t q = tid; q < nchunk; q += kSampleThreads) {
        const uint32_t first = sm.chunk_ties[q];
        const uint32_t next = q + 1 < nchunk ? sm.chunk_ties[q + 1] : total;
        if (next == first || first >= ties) continue;  // no ties here, or none of them in the support
        float x[8];
        load_chunk(rowp, vec, q, V, x);
        uint32_t rank = first;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          bool any = false;
#pragma unroll
          for (int i = 0; i < 4; ++i) any |= x[4 * b + i] == thr;
          if (!any) continue;
          const Ctr r = block_ctr(q, b);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (!(x[4 * b + i] == thr)) continue;
            if (rank < ties) f(x[4 * b + i], ctr_word(r, i), 8 * q + 4 * b + i);
            ++rank;
          }
        }
      }
      return;
    }
    uint32_t base = 0;
    int buf = 1;
    for (int64_t q0 = 0; q0 < nchunk && base < ties; q0 += kSampleThreads, buf ^= 1) {
      const int64_t q = q0 + tid;
      float x[8];
      uint32_t m = 0;
      if (q < nchunk) {
        load_chunk(rowp, vec, q, V, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) m |= (x[i] == thr ? 1u : 0u) << i;
      }
      uint32_t total;
      uint32_t rank = base + block_excl_scan(__builtin_popcount(m), total, sm, buf);
      if (m) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const uint32_t mb = (m >> (4 * b)) & 0xFu;
          if (!mb) continue;
          const Ctr r = block_ctr(q, b);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (!((mb >> i) & 1u)) continue;
            if (rank < ties) f(x[4 * b + i], ctr_word(r, i), 8 * q + 4 * b + i);
            ++rank;
          }
        }
      }
      base += total;
    }
  };

  // ---- pass 1: fp32 score intervals of every support candidate (a token at
  // -inf has probability 0 and is never drawn) ----
  Top1 gt = top1_empty(V), eq = top1_empty(V);
  auto track = [&](Top1& t) {
    return [&t, &d](float x, uint32_t r, int64_t id) {
      if (x == -__builtin_inff()) return;
      float err;
      const float s32 = score32(x, r, d, err);
      top1_add(t, s32, err, int32_t(id));
    };
  };
  const uint32_t n_eq = each_token(true, track(gt), track(eq));
  uint32_t n_eq_total;
  (void)block_excl_scan(n_eq, n_eq_total, sm, 0);
  const bool partial = n_eq_total > ties;
  if (partial) {  // ---- pass 2: only the first `ties` threshold-equal tokens by id ----
    eq = top1_empty(V);
    each_ranked_tie(track(eq));
  }

  // ---- the decision in fp64, over the tokens that can still be the best ----
  const float L = block_max_f(fmaxf(gt.max_lo, eq.max_lo), sm);
  const float over = block_max_f((gt.b2 >= L || eq.b2 >= L) ? 1.0f : 0.0f, sm);
  Best best{-__builtin_inf(), int64_t(V)};
  auto exact = [&](float x, uint32_t r, int64_t id) {
    if (x == -__builtin_inff()) return;
    float err;
    const float s32 = score32(x, r, d, err);
    if (!(s32 + err >= L)) return;
    const Best c{gumbel_score(x, r, d), id};
    if (better(c, best)) best = c;
  };
  if (over == 0.0f) {
    const Top1* ts[2] = {&gt, &eq};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const Top1& t = *ts[k];
      if (t.id1 < V && t.hi1 >= L) {
        const int64_t id = t.id1;
        const Ctr r = block_ctr(id >> 3, int((id >> 2) & 1));
        exact(bf16_to_f32(rowp[id]), ctr_word(r, int(id & 3)), id);
      }
    }
  } else {  // some token not kept may be a winner: rescan the row in the exact mode (rare)
    if (partial) {
      each_token(false, exact, [](float, uint32_t, int64_t) {});
      each_ranked_tie(exact);
    } else {
      each_token(false, exact, exact);
    }
  }
  best = block_best(best, sm);
  if (tid == 0) sampled[row] = best.id;
}

// The order in which sample_kernel takes its rows: the largest supports first.
// A row's cost grows with its support (a Philox block and two logarithms per
// support token, on top of one read of the row), and a whole-vocabulary
// support costs tens of times a small one; rows taken in index order leave
// the last large ones running alone at the end of the grid.  One workgroup:
// rows go to kOrderBuckets buckets by support size (bad rows last), the
// buckets are laid out largest first, and each row takes the next place in
// its bucket (the order inside a bucket is whatever the atomics give: every
// row is drawn independently of the others).
constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = 5;
__device__ __forceinline__ int support_bucket(int32_t len, uint8_t st) {
  if (st & kRowBad) return kOrderBuckets - 1;
  return len >= 65536 ? 0 : len >= 16384 ? 1 : len >= 4096 ? 2 : len >= 1024 ? 3 : 4;
}
__global__ __launch_bounds__(kOrderThreads) void order_rows_kernel(const int32_t* __restrict__ support_len,
                                                                   const uint8_t* __restrict__ status, int64_t rows,
                                                                   int32_t* __restrict__ order) {
  __shared__ uint32_t cnt[kOrderBuckets], place[kOrderBuckets];
  const int tid = threadIdx.x;
  if (tid < kOrderBuckets) cnt[tid] = 0u;
  __syncthreads();
  for (int64_t r = tid; r < rows; r += kOrderThreads) atomicAdd(&cnt[support_bucket(support_len[r], status[r])], 1u);
  __syncthreads();
  if (tid == 0) {
    uint32_t b = 0;
    for (int i = 0; i < kOrderBuckets; ++i) {
      place[i] = b;
      b += cnt[i];
    }
  }
  __syncthreads();
  for (int64_t r = tid; r < rows; r += kOrderThreads)
    order[atomicAdd(&place[support_bucket(support_len[r], status[r])], 1u)] = int32_t(r);
}

}  // namespace

int launch_order_rows(const int32_t* support_len, const uint8_t* status, int64_t rows, int32_t* order,
                      void* stream) {
  if (rows <= 0) return 0;
  order_rows_kernel<<<dim3(1), dim3(kOrderThreads), 0, static_cast<hipStream_t>(stream)>>>(support_len, status, rows,
                                                                                          order);
  return int(hipGetLastError());
}

int launch_sample(const uint16_t* logits, int64_t ld, int64_t rows, int64_t V, const float* temp, float temp_scalar,
                  const uint8_t* status, const float* threshold_logit, const int32_t* threshold_ties,
                  const float* row_max, uint64_t seed, uint64_t offset, int64_t* sampled, uint8_t* out_status,
                  int64_t row0, const int32_t* order, const int64_t* ids, int64_t cap, const int32_t* support_len,
                  void* stream) {
  if (rows <= 0) return 0;
  if (ids && (cap < 1 || cap > 64 || !support_len)) return int(hipErrorInvalidValue);
  sample_kernel<<<dim3(unsigned(rows)), dim3(kSampleThreads), 0, static_cast<hipStream_t>(stream)>>>(
      logits, ld, int(V), temp, temp_scalar, status, threshold_logit, threshold_ties, row_max, seed, offset, sampled,
      out_status, row0, order, ids, int(cap), support_len);
  return int(hipGetLastError());
}

}  // namespace vs

// Sampling-transform support and support-conditioned scores over bf16 logits.
//
// The program of xorl issue #71 section 3: temperature, then stable token-id
// top-k, inclusive top-p on the top-k renormalised masses, min-p against the
// original row max.  Rank order is (logit descending, token id ascending);
// each filter keeps a prefix of it, so the support is the shortest prefix
// pi[0:L].  Its scores follow SkyRL PR #2004 (renormalise over the support).
//
// Tokens are compared through 16-bit order-preserving keys (a larger key is a
// larger logit; -0 is folded onto +0).  Every token with the same key has the
// same probability, so every cut position and every support sum follows
// exactly from the histogram of key counts:
//   * 1024 segments of 64 keys, each with its token count, its mass
//     sum c * exp(z - z_max) and sum c * exp(z - z_max) * (z - z_max) in fp64
//     (a segment's weights form a geometric sequence: three exp calls);
//   * rank and mass queries walk the segments in descending key order, then
//     the 64 keys of one segment;
//   * inside the threshold key, ties go by token id: the support holds its
//     first r tokens.
// The histogram is 65536 16-bit counters packed two per LDS word (one
// branch-free atomic per token).  A counter that would pass 65535 (a key
// repeated that often) is detected from the exact total and the row is handed
// to the stream kernel, which re-reads the row for every pass and counts with
// 32-bit bins in two halves.
// Kernels:
//   * rows up to 20 * 512 * 8 tokens: one 512-thread workgroup per row with
//     the row in registers (transforms_fast_kernel<NV>);
//   * longer rows: a count kernel (1024 threads per row: histogram, checks,
//     per-row record of the non-empty counts and the dense-id candidates) and
//     a finish kernel (256 threads per row, four rows per CU: sums, cuts,
//     descriptor, dense ids, scores), or, above 2048 dense ids, one
//     1024-thread workgroup per row (transforms_fast_kernel<0>).
// Dense support ids come from ranking the few candidate tokens in LDS.  All
// sums run in a fixed order, so results are bitwise reproducible.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace vs {

namespace {

constexpr int NT = 512;          // threads of the register-resident kernels (row in registers)
constexpr int NT_STREAM = 1024;  // threads of the streaming kernels (row re-read from memory)
constexpr int MAX_WAVES = NT_STREAM / 64;

constexpr int HALF = 32768;
constexpr int SEGW = 64;
constexpr int NSEG = 65536 / SEGW;       // 1024
constexpr int COLLECT_MAX = 4096;
// Split path (streamed rows): a count kernel, then a finish kernel with
// NT_FIN threads and a candidate buffer of COLLECT_SPLIT entries, so that
// several rows share a CU.  The count kernel writes one record per row:
//   [kRecHead]   u32 kmax, candidate entries, K_cap, non-empty segments n;
//                then u32 candidate kind (kCandTokens / kCandUnits)
//   [kRecList]   u16[NSEG]: the n non-empty segments, descending
//   [kRecCand]   u64[COLLECT_SPLIT] candidate entries: tokens (key << 32 |
//                ~column), or units (vector index of the first 8 tokens |
//                vector index of the second 8, or ~0, << 32)
//   [kRecBlocks] u32[kRecMaxSegs][32]: the packed count words of list entry e
//                at e
// A row with more than kRecMaxSegs non-empty segments (keys spread over more
// than a quarter of the 1024 segments: bf16 logits of ordinary rows fill a
// few dozen) is handed to the stream kernel, as a counter overflow is, so the
// record is sized for what ordinary rows write.
constexpr int NT_FIN = 256;
constexpr int COLLECT_SPLIT = 2048;
constexpr int kRecMaxSegs = 256;
constexpr size_t kRecHead = 0, kRecList = 256, kRecCand = kRecList + size_t(NSEG) * 2;
constexpr uint32_t kCandTokens = 1, kCandUnits = 2;
constexpr size_t kRecBlocks = kRecCand + size_t(COLLECT_SPLIT) * 8;
constexpr size_t kRecBytes = kRecBlocks + size_t(kRecMaxSegs) * 128;
static_assert(kRecBytes % 256 == 0, "records stay 256-byte aligned");
constexpr uint32_t KEY_NEG_INF = 0x007Fu;
constexpr int kInFlight = 4;  // 16-byte loads per thread in flight in a streaming pass (1024 threads)

struct alignas(16) Smem {
  uint32_t hist[HALF];  // packed 16-bit counters (fast) or one half of 32-bit bins (stream); later candidates
  uint32_t seg_count[NSEG];
  double seg_mass[NSEG];
  double seg_zmass[NSEG];
  uint32_t fine[SEGW];  // 32-bit counts of one segment (stream kernel)
  uint32_t red_u[MAX_WAVES], red_v[MAX_WAVES];
  double red_m[MAX_WAVES], red_z[MAX_WAVES];
  uint32_t bu[8];  // broadcast slots (integers)
  double bd[8];    // broadcast slots (fp64)
  int fine_seg;
  uint32_t ncand;
  uint32_t zero_overflow;  // the -0 / +0 merge of the streaming count passed 16 bits
  __device__ uint64_t* cand_area() { return reinterpret_cast<uint64_t*>(hist); }
};
// The finish kernel's LDS (about 39 KiB: four rows per CU).  The first
// FIN_STAGED non-empty segments' count words are kept in LDS for the key
// queries, in the space the dense-id candidates use afterwards.
constexpr int FIN_STAGED = COLLECT_SPLIT * 2 / 32;  // 128 segments of 32 words
struct alignas(16) SmemFin {
  union {
    uint64_t cand[COLLECT_SPLIT];
    uint32_t blk[FIN_STAGED][32];
  };
  uint8_t seg_slot[NSEG];   // staging slot of a segment, 0xFF = not staged
  uint16_t nelist[NSEG];    // the non-empty segments, ascending
  uint32_t n_ne;
  uint32_t seg_count[NSEG];
  double seg_mass[NSEG];
  double seg_zmass[NSEG];
  uint32_t fine[SEGW];
  uint32_t red_u[MAX_WAVES];
  double red_m[MAX_WAVES], red_z[MAX_WAVES];
  uint32_t bu[8];
  double bd[8];
  int fine_seg;
  uint32_t ncand;
  __device__ uint64_t* cand_area() { return cand; }
};

// raw bf16 pattern -> order-preserving key (-0 folded onto +0)
__device__ __forceinline__ uint32_t key16(uint32_t h) {
  h = (h & 0x7FFFu) ? h : 0u;
  return (h & 0x8000u) ? (h ^ 0xFFFFu) : (h | 0x8000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  const uint32_t h = (k & 0x8000u) ? (k & 0x7FFFu) : (k ^ 0xFFFFu);
  return __uint_as_float(h << 16);
}
__device__ __forceinline__ bool raw_bad(uint32_t h) { return (h & 0x7FFFu) >= 0x7F80u && h != 0xFF80u; }

// Packed 16-bit helpers for the count pass (one VALU op per 32-bit word).
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// the keys of both bf16 halves of a word, -0 left at 0x7FFF: a per-half
// arithmetic shift by 15 gives 0xFFFF where the sign is set and 0 elsewhere,
// so the xor mask is that or 0x8000 (sign set: h ^ 0xFFFF, clear: h ^ 0x8000)
__device__ __forceinline__ uint32_t pair_keys(uint32_t w) {
  const s16x2 smear = __builtin_bit_cast(s16x2, w) >> 15;
  return w ^ (__builtin_bit_cast(uint32_t, smear) | 0x80008000u);
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(
      uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// Inclusive prefix sums across the 64 lanes of a wave with DPP moves (no LDS
// traffic, unlike lane shuffles): shifts by 1, 2, 4, 8 inside each row of 16
// lanes (lanes shifted in from outside a row read 0), then lane 15 of rows 0
// and 2 added into rows 1 and 3, then lane 31 into rows 2 and 3.  A fixed
// order, so results are reproducible.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xf, true));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = __builtin_bit_cast(unsigned long long, v);
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>(uint32_t(b)), hi = dpp_u32<CTRL, ROW_MASK>(uint32_t(b >> 32));
  return __builtin_bit_cast(double, (static_cast<unsigned long long>(hi) << 32) | lo);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
template <class T, class Move, class Op>
__device__ __forceinline__ T wave_scan_incl(T x, Move mv, Op op) {
  x = op(x, mv(x, std::integral_constant<int, kRowShr1>{}, std::integral_constant<int, 0xf>{}));
  x = op(x, mv(x, std::integral_constant<int, kRowShr2>{}, std::integral_constant<int, 0xf>{}));
  x = op(x, mv(x, std::integral_constant<int, kRowShr4>{}, std::integral_constant<int, 0xf>{}));
  x = op(x, mv(x, std::integral_constant<int, kRowShr8>{}, std::integral_constant<int, 0xf>{}));
  x = op(x, mv(x, std::integral_constant<int, kRowBcast15>{}, std::integral_constant<int, 0xa>{}));
  x = op(x, mv(x, std::integral_constant<int, kRowBcast31>{}, std::integral_constant<int, 0xc>{}));
  return x;
}
struct AddOp {
  template <class T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
__device__ __forceinline__ uint32_t wave_scan_incl_u32(uint32_t x) {
  return wave_scan_incl(
      x, [](uint32_t v, auto c, auto m) { return dpp_u32<decltype(c)::value, decltype(m)::value>(v); }, AddOp{});
}
// the wave's total / maximum (a running maximum with 0 for lanes shifted in
// from outside a row: the identity for unsigned values), read from lane 63
__device__ __forceinline__ uint32_t wave_total_u32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_readlane(int(wave_scan_incl_u32(x)), 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  const uint32_t r = wave_scan_incl(
      x, [](uint32_t v, auto c, auto m) { return dpp_u32<decltype(c)::value, decltype(m)::value>(v); },
      [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  return uint32_t(__builtin_amdgcn_readlane(int(r), 63));
}
__device__ __forceinline__ double wave_scan_incl_f64(double x) {
  return wave_scan_incl(
      x, [](double v, auto c, auto m) { return dpp_f64<decltype(c)::value, decltype(m)::value>(v); }, AddOp{});
}

template <int NW, class SM>
__device__ uint32_t block_sum_u32(uint32_t v, SM& sm) {
  v = wave_total_u32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.red_u[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += sm.red_u[i];
  return t;
}
template <int NW, class SM>
__device__ uint32_t block_max_u32(uint32_t v, SM& sm) {
  v = wave_max_u32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.red_u[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t = max(t, sm.red_u[i]);
  return t;
}
// Exclusive prefix over threads in thread order; also returns the total.
template <int NW, class SM>
__device__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t& total, SM& sm) {
  const int lane = threadIdx.x & 63;
  const uint32_t incl = wave_scan_incl_u32(v);
  __syncthreads();
  if (lane == 63) sm.red_u[threadIdx.x >> 6] = incl;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t t = sm.red_u[i];
    if (i < int(threadIdx.x >> 6)) before += t;
    total += t;
  }
  return before + incl - v;
}

// Two exclusive scans at once (the same barriers).
template <int NW, class SM>
__device__ void block_excl_scan2_u32(uint32_t v, uint32_t w, uint32_t& ev, uint32_t& ew, uint32_t& tv, uint32_t& tw,
                                     SM& sm) {
  const int lane = threadIdx.x & 63;
  const uint32_t iv = wave_scan_incl_u32(v), iw = wave_scan_incl_u32(w);
  __syncthreads();
  if (lane == 63) {
    sm.red_u[threadIdx.x >> 6] = iv;
    sm.red_v[threadIdx.x >> 6] = iw;
  }
  __syncthreads();
  uint32_t bv = 0, bw = 0;
  tv = tw = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t a = sm.red_u[i], b = sm.red_v[i];
    if (i < int(threadIdx.x >> 6)) {
      bv += a;
      bw += b;
    }
    tv += a;
    tw += b;
  }
  ev = bv + iv - v;
  ew = bw + iw - w;
}

// ---------------------------------------------------------------------------
// Key sources.  each(f) calls f(key, column) for every token of this thread
// (register keys also visit padding columns, whose key 0 lies below every
// real key); slice(j, f) does the same for slice j, slices being in column
// order and, inside a slice, columns increasing with (thread, position).
// ---------------------------------------------------------------------------
template <int NV>
struct RegKeys {
  uint32_t kw[NV][4];  // two keys per word
  static constexpr int kThreads = NT;
  static constexpr int kCollectMax = COLLECT_MAX;
  static constexpr bool kTopList = false;  // the row is in registers: a sweep is cheap
  struct Listed {};
  __device__ __forceinline__ bool listed_from(uint32_t) const { return false; }
  __device__ __forceinline__ Listed load_listed() const { return Listed{}; }
  template <class F>
  __device__ __forceinline__ void each_listed(const Listed&, uint32_t, F) const {}

  // Loads the row, converts it to keys and counts every key into the packed
  // 16-bit counters `hist` (already zeroed); returns bad (NaN or +inf seen)
  // and this thread's max key.  Vectors go in groups of 8 (128 bytes per
  // thread in flight): each group is loaded, converted and counted before the
  // next, which bounds the registers the unrolled loop needs.
  __device__ __forceinline__ void load_count(const uint16_t* rowp, int V, uint32_t* hist, uint32_t& bad,
                                             uint32_t& kmax) {
    const int tid = threadIdx.x;
    const bool aligned = (reinterpret_cast<uintptr_t>(rowp) & 15) == 0;
    bad = 0;
    kmax = 0;
    constexpr int G = 8;
#pragma unroll
    for (int g = 0; g < NV; g += G) {
      uint32_t wv[G][4];
#pragma unroll
      for (int jj = 0; jj < G && g + jj < NV; ++jj) {
        const int q = tid + NT * (g + jj);
        if (aligned && 8 * q + 8 <= V) {
          const uint4 v = reinterpret_cast<const uint4*>(rowp)[q];
          wv[jj][0] = v.x;
          wv[jj][1] = v.y;
          wv[jj][2] = v.z;
          wv[jj][3] = v.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c0 = 8 * q + 2 * e;
            // padding columns get the raw pattern 0xFFFF, whose key is 0
            const uint32_t lo = c0 < V ? uint32_t(rowp[c0]) : 0xFFFFu;
            const uint32_t hi = c0 + 1 < V ? uint32_t(rowp[c0 + 1]) : 0xFFFFu;
            wv[jj][e] = lo | (hi << 16);
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < G && g + jj < NV; ++jj) {
        const int q = tid + NT * (g + jj);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t w = wv[jj][e];
          const uint32_t lo = w & 0xFFFFu, hi = w >> 16;
          const int c0 = 8 * q + 2 * e;
          bad |= (c0 < V && raw_bad(lo)) ? 1u : 0u;
          bad |= (c0 + 1 < V && raw_bad(hi)) ? 1u : 0u;
          // -0 -> +0; then negative halves invert all 16 bits, positive ones set the top bit
          w &= ~(((lo & 0x7FFFu) ? 0u : 0x8000u) | ((hi & 0x7FFFu) ? 0u : 0x80000000u));
          const uint32_t neg = ((w >> 15) & 0x00010001u) * 0xFFFFu;
          w ^= neg | 0x80008000u;
          kw[g + jj][e] = w;
          const uint32_t k0 = w & 0xFFFFu, k1 = w >> 16;
          kmax = max(kmax, max(k0, k1));
          atomicAdd(&hist[k0 >> 1], (k0 & 1u) ? 0x10000u : 1u);
          atomicAdd(&hist[k1 >> 1], (k1 & 1u) ? 0x10000u : 1u);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // An empty asm that claims to rewrite every packed word: values unpacked in
  // an earlier pass cannot be reused, so the unpacked keys (twice the
  // registers) never stay live across the kernel.  No instruction is emitted.
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(kw[j][e]));
  }
  template <class F>
  __device__ __forceinline__ void each(F f) {
    opaque();
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      slice(j, f);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __device__ __forceinline__ int slices() const { return NV; }
  template <class F>
  __device__ __forceinline__ void slice(int j, F f) const {
    const int c0 = 8 * (int(threadIdx.x) + NT * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f(kw[j][e] & 0xFFFFu, c0 + 2 * e);
      f(kw[j][e] >> 16, c0 + 2 * e + 1);
    }
  }
};

template <int NTH_>
struct StreamKeysT {
  const uint16_t* rowp;
  int V;
  // The count pass visits vector q (logical) at vector phys(q) = (q + rot) mod
  // nvec: rows read at once start at different offsets (one contiguous stream
  // per row, all from offset 0, camps on a subset of the memory channels).
  int rot;
  // Filled by load_count.  The thread's 8-token vectors q and q + kThreads
  // form a unit (the second absent past the last whole vector).  Kept: the
  // thread's two best units by their largest key (first vector index, -1 =
  // none) and the largest key of every token outside them, so every token
  // with a key above `dropped` is in the listed units.  Tail tokens (past the
  // last whole vector) always count as dropped.
  uint32_t vkey[2];
  int vq[2];
  uint32_t dropped;
  bool have_top;
  static constexpr int kThreads = NTH_;
  static constexpr int kCollectMax = COLLECT_MAX;
  static constexpr bool kTopList = true;
  __device__ __forceinline__ void opaque() {}
  __device__ __forceinline__ bool aligned() const { return (reinterpret_cast<uintptr_t>(rowp) & 15) == 0; }
  __device__ __forceinline__ int nvec() const { return aligned() ? V / 8 : 0; }
  __device__ __forceinline__ int phys(int q, int nv) const {
    const int p = q + rot;
    return p < nv ? p : p - nv;
  }
  // branch-free update of the two-unit list with unit q of largest key vmax
  __device__ __forceinline__ void offer_vector(uint32_t vmax, int q) {
    const bool in0 = vmax > vkey[0];
    const bool in1 = vmax > vkey[1];
    dropped = max(dropped, in1 ? vkey[1] : vmax);  // the unit that leaves (or never enters)
    const uint32_t k1 = in0 ? vkey[0] : (in1 ? vmax : vkey[1]);
    const int q1 = in0 ? vq[0] : (in1 ? q : vq[1]);
    vkey[0] = in0 ? vmax : vkey[0];
    vq[0] = in0 ? q : vq[0];
    vkey[1] = k1;
    vq[1] = q1;
  }
  // true when every token of this thread with key >= K is in the listed units
  __device__ __forceinline__ bool listed_from(uint32_t K) const { return have_top && dropped < K; }
  struct Listed {
    uint4 v[4];
  };
  // The data of the listed units whose largest key is >= K (the others are
  // not loaded: by the end of the count their lines have left the caches,
  // and a scattered 16-byte piece costs a whole line from memory).
  __device__ __forceinline__ Listed issue_listed(uint32_t K) const {
    const uint4* pv = reinterpret_cast<const uint4*>(rowp);
    const int nv = nvec();
    Listed l;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = vq[i];
      const bool use = q >= 0 && vkey[i] >= K;
      l.v[2 * i] = use ? pv[phys(q, nv)] : make_uint4(0, 0, 0, 0);
      l.v[2 * i + 1] = (use && q + kThreads < nv) ? pv[phys(q + kThreads, nv)] : make_uint4(0, 0, 0, 0);
    }
    return l;
  }
  __device__ __forceinline__ Listed load_listed() const { return issue_listed(0); }
  // f(key, column) for the listed tokens, possibly skipping tokens with key < K:
  // a unit whose largest key is below K is skipped, and so is a word whose
  // larger raw key is below K - 1 (-0 sits one below +0 before the fold)
  template <class F>
  __device__ __forceinline__ void each_listed(const Listed& l, uint32_t K, F f) const {
    const int nv = nvec();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = vq[i] + h * kThreads;
        const bool ok = vq[i] >= 0 && q < nv && vkey[i] >= K;
        const int c0 = 8 * (ok ? phys(q, nv) : 0);
        const uint4 v = l.v[2 * i + h];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t keys = pair_keys(w[e]);
          if (ok && max(keys & 0xFFFFu, keys >> 16) + 1u >= K) {
            f(key16(w[e] & 0xFFFFu), c0 + 2 * e);
            f(key16(w[e] >> 16), c0 + 2 * e + 1);
          }
        }
      }
    }
  }
  // Count every token into the packed histogram and track the row's largest
  // key (and, through it, NaN / +inf).  Negative NaNs (keys <= 0x7E) are found
  // afterwards from the histogram's lowest bins (low_bad).
  // The count pass's first batch of loads (this thread's vectors q = t,
  // t + kThreads, ...), issued ahead so they stream during other work.
  __device__ __forceinline__ void prefetch(uint4 (&v)[kInFlight]) const {
    const int nv = nvec();
    const uint4* pv = reinterpret_cast<const uint4*>(rowp);
    const int q = threadIdx.x;
    if (q + (kInFlight - 1) * kThreads < nv) {
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) v[u] = pv[phys(q + u * kThreads, nv)];
    }
  }
  __device__ __forceinline__ void load_count(uint32_t* hist, uint32_t& kmax) {
    uint4 first[kInFlight];
    prefetch(first);
    load_count(hist, kmax, first);
  }
  // `first` holds what prefetch() loaded for this row.
  __device__ __forceinline__ void load_count(uint32_t* hist, uint32_t& kmax, const uint4 (&first)[kInFlight]) {
    kmax = 0;
    vkey[0] = vkey[1] = 0;
    vq[0] = vq[1] = -1;
    dropped = 0;
    have_top = true;
    // Key k counts in the 16-bit half (k & 1) of word k >> 1: byte 2 (k & ~1),
    // increment 1 << 16 (k & 1).  Both halves' addresses and shift counts come
    // from the packed keys with one op each (16-bit halves read by word
    // select).  -0 keeps its key 0x7FFF here: its count is merged into +0's
    // (0x8000) once counting is done (merge_zero), and a unit's largest key is
    // folded below, which is all the candidate lists and the row max need.
    char* const hb = reinterpret_cast<char*>(hist);
    auto pair = [&](uint32_t w) -> uint32_t {
      const uint32_t keys = pair_keys(w);
      const uint32_t even = keys & 0xFFFEFFFEu;
      const uint32_t sh = (keys & 0x00010001u) << 4;
      atomicAdd(reinterpret_cast<uint32_t*>(hb + ((even & 0xFFFFu) << 1)), 1u << (sh & 0xFFFFu));
      atomicAdd(reinterpret_cast<uint32_t*>(hb + ((even >> 16) << 1)), 1u << (sh >> 16));
      return keys;
    };
    auto vec_max = [&](const uint4& v) -> uint32_t {
      return pk_max_u16(pk_max_u16(pair(v.x), pair(v.y)), pk_max_u16(pair(v.z), pair(v.w)));
    };
    auto unit = [&](uint32_t hi, int qv) {
      uint32_t vmax = max(hi & 0xFFFFu, hi >> 16);
      vmax = vmax == 0x7FFFu ? 0x8000u : vmax;
      kmax = max(kmax, vmax);
      offer_vector(vmax, qv);
    };
    constexpr int nt = kThreads;
    const int nv = nvec();
    const uint4* pv = reinterpret_cast<const uint4*>(rowp);
    int q = threadIdx.x;
    static_assert(kInFlight % 2 == 0, "units are vector pairs");
    if (q + (kInFlight - 1) * nt < nv) {
#pragma unroll
      for (int u = 0; u < kInFlight; u += 2) unit(pk_max_u16(vec_max(first[u]), vec_max(first[u + 1])), q + u * nt);
      q += kInFlight * nt;
    }
    for (; q + (kInFlight - 1) * nt < nv; q += kInFlight * nt) {
      uint4 v[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) v[u] = pv[phys(q + u * nt, nv)];
#pragma unroll
      for (int u = 0; u < kInFlight; u += 2) unit(pk_max_u16(vec_max(v[u]), vec_max(v[u + 1])), q + u * nt);
    }
    for (; q + nt < nv; q += 2 * nt) unit(pk_max_u16(vec_max(pv[phys(q, nv)]), vec_max(pv[phys(q + nt, nv)])), q);
    if (q < nv) unit(vec_max(pv[phys(q, nv)]), q);
    for (int c = 8 * nv + int(threadIdx.x); c < V; c += nt) {
      const uint32_t k = key16(rowp[c]);
      count(hist, k);
      kmax = max(kmax, k);
      dropped = max(dropped, k);
    }
  }
  __device__ __forceinline__ static void count(uint32_t* hist, uint32_t k) {
    atomicAdd(&hist[k >> 1], (k & 1u) ? 0x10000u : 1u);
  }
  // After counting: whether any key <= 0x7E (a negative NaN; -inf is 0x7F)
  // was counted, from the 64 lowest words (one per thread of wave 0).
  __device__ __forceinline__ static bool low_bad(const uint32_t* hist, int tid) {
    return tid < 64 && (hist[tid] & (tid == 0x3F ? 0xFFFFu : 0xFFFFFFFFu)) != 0;
  }
  // After counting: move the tokens counted under -0's key (0x7FFF, high half
  // of word 0x3FFF) to +0's (0x8000, low half of word 0x4000).  Returns false
  // when the merged count does not fit 16 bits.  One thread.
  __device__ __forceinline__ static bool merge_zero(uint32_t* hist) {
    const uint32_t w1 = hist[0x3FFF], w2 = hist[0x4000];
    const uint32_t a = w1 >> 16, b = w2 & 0xFFFFu;
    if (a == 0) return true;
    if (a + b > 0xFFFFu) return false;
    hist[0x3FFF] = w1 & 0xFFFFu;
    hist[0x4000] = (w2 & 0xFFFF0000u) | (a + b);
    return true;
  }
  template <class F>
  __device__ __forceinline__ void each(F f) const {
    constexpr int nt = kThreads;
    const int nvec = aligned() ? V / 8 : 0;
    const uint4* pv = reinterpret_cast<const uint4*>(rowp);
    int q = threadIdx.x;
    for (; q + (kInFlight - 1) * nt < nvec; q += kInFlight * nt) {
      uint4 v[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) v[u] = pv[q + u * nt];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        const int c0 = 8 * (q + u * nt);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f(key16(w[e] & 0xFFFFu), c0 + 2 * e);
          f(key16(w[e] >> 16), c0 + 2 * e + 1);
        }
      }
    }
    for (; q < nvec; q += nt) {
      const uint4 v = pv[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f(key16(w[e] & 0xFFFFu), 8 * q + 2 * e);
        f(key16(w[e] >> 16), 8 * q + 2 * e + 1);
      }
    }
    for (int c = 8 * nvec + int(threadIdx.x); c < V; c += nt) f(key16(rowp[c]), c);
  }
  __device__ __forceinline__ int slices() const { return (V + kThreads - 1) / kThreads; }
  template <class F>
  __device__ __forceinline__ void slice(int j, F f) const {
    const int c = int(threadIdx.x) + kThreads * j;
    if (c < V) f(key16(rowp[c]), c);
  }
};
using StreamKeys = StreamKeysT<NT_STREAM>;

// The finish kernel's view of a row: sweeps re-read it with NT_FIN threads;
// the listed candidates are the ones the count kernel stored: every token with
// key >= K_cap (the dense-id cut is never below it), when there are no more
// than COLLECT_SPLIT of them.
// The finish kernel's first candidate entry of thread t: consecutive entries
// go to different waves, so a row's few candidates spread over all four.
__device__ __forceinline__ uint32_t fin_entry(int t) { return uint32_t(((t & 63) << 2) | (t >> 6)); }
static_assert(NT_FIN == 256, "fin_entry spreads entries over four waves");

struct SplitKeys : StreamKeysT<NT_FIN> {
  const uint64_t* cand_g;
  uint64_t cand0;  // this thread's first candidate entry, loaded early
  uint4 unit0[2];  // its data when the entries are units (loaded early too)
  uint32_t ncand_g;
  uint32_t kind;   // kCandTokens or kCandUnits
  static constexpr int kCollectMax = COLLECT_SPLIT;
  struct Listed {};
  __device__ __forceinline__ Listed load_listed() const { return Listed{}; }
  __device__ __forceinline__ bool listed_from(uint32_t) const { return ncand_g <= uint32_t(COLLECT_SPLIT); }
  // the two 8-token vectors of unit entry e (the second absent: zeros)
  __device__ __forceinline__ void load_unit(uint64_t e, uint4 (&u)[2]) const {
    const uint4* pv = reinterpret_cast<const uint4*>(rowp);
    const uint32_t v0 = uint32_t(e & 0xFFFFFFFFu), v1 = uint32_t(e >> 32);
    u[0] = pv[v0];
    u[1] = v1 != 0xFFFFFFFFu ? pv[v1] : make_uint4(0, 0, 0, 0);
  }
  template <class F>
  __device__ __forceinline__ void each_listed(const Listed&, uint32_t, F f) const {
    const uint32_t first = fin_entry(threadIdx.x);
    for (uint32_t i = first; i < ncand_g; i += kThreads) {
      const uint64_t e = i == first ? cand0 : cand_g[i];
      if (kind == kCandTokens) {
        f(uint32_t(e >> 32), int(0xFFFFFFFFu - uint32_t(e & 0xFFFFFFFFu)));
        continue;
      }
      uint4 u[2];
      if (i == first) {
        u[0] = unit0[0];
        u[1] = unit0[1];
      } else {
        load_unit(e, u);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t v = h == 0 ? uint32_t(e & 0xFFFFFFFFu) : uint32_t(e >> 32);
        if (v == 0xFFFFFFFFu) continue;
        const uint32_t w[4] = {u[h].x, u[h].y, u[h].z, u[h].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f(key16(w[k] & 0xFFFFu), int(8 * v + 2 * k));
          f(key16(w[k] >> 16), int(8 * v + 2 * k + 1));
        }
      }
    }
  }
};

// z - z_max of key k in fp64, from the exact difference of the two logits
// (bf16 values are exact in fp64), divided by tau once.  Forming x / tau - z_max
// instead would carry a rounding error of about |x / tau| * 2^-53, which at
// large magnitudes is far from small once exponentiated.
__device__ __forceinline__ double key_d(uint32_t k, double tau, double xmax) {
  return (double(key_logit(k)) - xmax) / tau;
}
// fp64 weight of a key relative to the row max: exp(z - z_max), the quantity
// the program compares with min_p and sums for the masses.
__device__ __forceinline__ double key_weight(uint32_t k, double tau, double xmax) {
  return exp(key_d(k, tau, xmax));
}

struct RowArgs {
  int64_t row;
  int V;
  float tauf;
  int kk;
  float pf, mpf;
  int64_t y;
  uint32_t key_y;  // key of the target's logit, loaded early
  const uint16_t* rowp;
  float* logprob;
  float* entropy;
  uint8_t* status;
  int32_t* support_len;
  float* threshold_logit;
  int32_t* threshold_ties;
  int64_t* ids_out;
  int cap;
  float* full_lse;
  float* row_max;  // the row's largest logit (nullable; the sampler's shift)
};

template <int NTH>
__device__ void write_bad(const RowArgs& a) {
  const float nanf = __builtin_nanf("");
  if (threadIdx.x == 0) {
    a.logprob[a.row] = nanf;
    if (a.entropy) a.entropy[a.row] = nanf;
    if (a.status) a.status[a.row] = kRowBad;
    if (a.support_len) a.support_len[a.row] = 0;
    if (a.threshold_logit) a.threshold_logit[a.row] = nanf;
    if (a.threshold_ties) a.threshold_ties[a.row] = 0;
    if (a.full_lse) a.full_lse[a.row] = nanf;
    if (a.row_max) a.row_max[a.row] = nanf;
  }
  if (a.ids_out)
    for (int i = threadIdx.x; i < a.cap; i += NTH) a.ids_out[a.row * a.cap + i] = -1;
}

__device__ __forceinline__ bool params_ok(const RowArgs& a) {
  return tau_ok(a.tauf) && (a.pf == a.pf) && a.pf > 0.0f && (a.mpf == a.mpf) && a.mpf <= 1.0f && a.y >= 0 &&
         a.y < a.V;
}

// Segment summary from the counts of its 64 keys (ascending key order).
template <class CountFn>
__device__ __forceinline__ void summarize_segment(int seg, CountFn count, double tau, double xmax, Smem& sm) {
  uint32_t cnt = 0;
  double mass = 0.0, zm = 0.0;
  for (int b = 0; b < SEGW; ++b) {
    const uint32_t key = uint32_t(seg * SEGW + b);
    const uint32_t c = count(key);
    if (c) {
      cnt += c;
      const double d = key_d(key, tau, xmax);
      const double e = exp(d);
      if (e > 0.0) {
        mass += double(c) * e;
        zm += double(c) * e * d;
      }
    }
  }
  sm.seg_count[seg] = cnt;
  sm.seg_mass[seg] = mass;
  sm.seg_zmass[seg] = zm;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) { return wave_total_u32(v); }

// The masses of regular segment s (2 .. NSEG-3, at least one key counted)
// from its 32 count words word(j) (keys 2j, 2j+1), visited from word rot on:
// the weights follow the geometric recurrence upwards from exp(d0).  That
// holds when every weight of the segment's keys, counted or not, is a normal
// number (-700 <= d <= 700 over the segment); otherwise (keys so far apart
// that the low weights underflow or, above the row max, overflow) nothing is
// added and false is returned: the caller then runs segment_masses_down.
template <class WordFn>
__device__ __forceinline__ bool segment_masses(int s, WordFn word, int rot, double tau, double xmax, double& m,
                                               double& zm) {
  const uint32_t k0 = uint32_t(s * SEGW);
  const double x0 = double(key_logit(k0));
  const double dd = (double(key_logit(k0 + 1)) - x0) / tau;  // exact spacing / tau
  const double d0 = (x0 - xmax) / tau;
  // the last key's offset from its own logit, not d0 + 63 dd: with huge
  // spacings that sum would carry the rounding of two huge terms
  const double d_last = key_d(k0 + uint32_t(SEGW - 1), tau, xmax);
  if (d_last < -746.0) return true;  // every weight is 0 in fp64
  if (d0 < -700.0 || d_last > 700.0) return false;
  const double r = exp(dd);
  const double r2 = r * r;
  const double w_first = exp(d0);
  double w = exp(d0 + double(2 * rot) * dd);  // weight of key 2 * rot
#pragma unroll 8
  for (int i = 0; i < 32; ++i) {
    const int j = (i + rot) & 31;
    if (i > 0 && j == 0) w = w_first;  // wrapped to the segment's first key
    const uint32_t wd = word(j);
    const double dl = d0 + double(2 * j) * dd;
    const double cl = double(wd & 0xFFFFu) * w;
    const double ch = double(wd >> 16) * (w * r);
    m += cl;
    m += ch;
    zm += cl * dl;
    zm += ch * (dl + dd);
    w *= r2;
  }
  return true;
}
// The same masses for the segments segment_masses declines (keys so far
// apart that a recurrence over them would overflow, underflow or carry the
// rounding of huge offsets): one exponential per counted key, from the top
// counted key down, each exponent taken from the key's own logit (key_d), so
// the row maximum has exactly weight 1 and z - z_max = 0.  Weights fall with
// the key, so the walk stops at the first weight that is 0; what it leaves out
// is below the fp64 resolution of the row's mass, which is at least 1.
template <class WordFn>
__device__ __forceinline__ void segment_masses_down(int s, WordFn word, double tau, double xmax, double& m,
                                                 double& zm) {
  const uint32_t k0 = uint32_t(s * SEGW);
  for (int k = SEGW - 1; k >= 0; --k) {
    const uint32_t c = (word(k >> 1) >> ((k & 1) * 16)) & 0xFFFFu;
    if (!c) continue;
    const double d = key_d(k0 + uint32_t(k), tau, xmax);
    const double w = exp(d);
    if (w == 0.0) break;
    const double ck = double(c) * w;
    m += ck;
    zm += ck * d;
  }
}

// All segment summaries in one pass, one thread per segment.  The thread
// loads the segment's 32 packed count words once (starting at word t % 32, so
// a wave's loads fall in different banks), adds up its token count and, for a
// non-empty regular segment (2 .. 1021: finite logits only), its masses
// sum c * exp(z - z_max) and sum c * exp(z - z_max) * (z - z_max) in fp64.
// The 64 keys of a regular segment are equally spaced logits (one exponent,
// consecutive mantissas), so w(key 2j) = exp(d_0) r^(2j) with r = exp(dx / tau):
// three exp calls per segment and a multiply per key pair.  The irregular
// segments hold only NaN and +-inf keys; in a row that passed the checks only
// -inf (weight 0) and the register paths' padding at key 0 can be counted.
// Returns this thread's share of the sum of all counts.
template <int NTH>
__device__ __forceinline__ uint32_t summarize_segments(const uint32_t* hist, uint32_t n_pad, double tau, double xmax,
                                                      Smem& sm) {
  uint32_t total = 0;
  const int rot = int(threadIdx.x & 31);
  uint32_t down = 0;  // bit i: this thread's i-th segment needs segment_masses_down
  int i = 0;
  for (int s = threadIdx.x; s < NSEG; s += NTH, ++i) {
    const uint32_t* seg = hist + s * 32;  // word j holds keys 2j (low half) and 2j + 1 (high half)
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t wd = seg[(i + rot) & 31];
      cnt += (wd & 0xFFFFu) + (wd >> 16);
    }
    if (s == 0) cnt -= n_pad;
    total += cnt;
    double m = 0.0, zm = 0.0;
    if (cnt != 0 && s >= 2 && s < NSEG - 2 && !segment_masses(s, [&](int j) { return seg[j]; }, rot, tau, xmax, m, zm))
      down |= 1u << i;
    sm.seg_count[s] = cnt;
    sm.seg_mass[s] = m;
    sm.seg_zmass[s] = zm;
  }
  if (down) {
    i = 0;
    for (int s = threadIdx.x; s < NSEG; s += NTH, ++i) {
      if (!((down >> i) & 1u)) continue;
      const uint32_t* seg = hist + s * 32;
      double m = 0.0, zm = 0.0;
      segment_masses_down(s, [&](int j) { return seg[j]; }, tau, xmax, m, zm);
      sm.seg_mass[s] = m;
      sm.seg_zmass[s] = zm;
    }
  }
  return total;
}

// Everything after the histogram: cuts, scores, descriptor, dense ids.
// `fine(s)` makes the 64 key counts of segment s readable through count(key).
template <class Keys, class FineFn, class CountFn, class SM>
__device__ void finish_row(const RowArgs& a, Keys& keys, uint32_t kmax, double tau, double xmax, SM& sm,
                           FineFn fine, CountFn count) {
  constexpr int NTH = Keys::kThreads;
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const bool w0 = tid < 64;

  // Segment prefixes in descending key order, in place: afterwards
  // seg_count[s] / seg_mass[s] / seg_zmass[s] hold the tokens / mass / z-mass
  // of all segments >= s.  Thread t owns descending positions SPT*t ..
  // SPT*t + SPT-1; a wave scan and a scan over the wave totals follow, all in
  // a fixed order (bitwise reproducible).
  {
    constexpr int SPT = NSEG / NTH;
    const int wave = tid >> 6;
    uint32_t c = 0;
    double m = 0.0, zm = 0.0;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int sg = NSEG - 1 - (SPT * tid + i);
      c += sm.seg_count[sg];
      m += sm.seg_mass[sg];
      zm += sm.seg_zmass[sg];
    }
    const uint32_t ci = wave_scan_incl_u32(c);
    const double mi = wave_scan_incl_f64(m), zi = wave_scan_incl_f64(zm);
    if (lane == 63) {
      sm.red_u[wave] = ci;
      sm.red_m[wave] = mi;
      sm.red_z[wave] = zi;
    }
    __syncthreads();
    uint32_t cw = 0;
    double mw = 0.0, zw = 0.0;
    for (int i = 0; i < wave; ++i) {
      cw += sm.red_u[i];
      mw += sm.red_m[i];
      zw += sm.red_z[i];
    }
    // exclusive start of this thread, then its own positions one by one
    c = cw + (ci - c);
    m = mw + (mi - m);
    zm = zw + (zi - zm);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int sg = NSEG - 1 - (SPT * tid + i);
      c += sm.seg_count[sg];
      m += sm.seg_mass[sg];
      zm += sm.seg_zmass[sg];
      sm.seg_count[sg] = c;
      sm.seg_mass[sg] = m;
      sm.seg_zmass[sg] = zm;
    }
  }
  __syncthreads();
  const double total_mass = sm.seg_mass[0];
  // tokens / mass / z-mass of the segments above s (s excluded)
  auto cnt_above = [&](int s) -> uint32_t { return s + 1 < NSEG ? sm.seg_count[s + 1] : 0u; };
  auto mass_above = [&](int s) -> double { return s + 1 < NSEG ? sm.seg_mass[s + 1] : 0.0; };
  auto zmass_above = [&](int s) -> double { return s + 1 < NSEG ? sm.seg_zmass[s + 1] : 0.0; };
  auto put_seg = [&](int s) {
    sm.bu[0] = uint32_t(s);
    sm.bu[1] = cnt_above(s);
    sm.bd[0] = mass_above(s);
    sm.bd[1] = zmass_above(s);
  };

  // Segment holding rank r (0-based, r < total): bu[0] = segment, bu[1] =
  // tokens above it, bd[0] / bd[1] = mass / z-mass above it.  One segment
  // satisfies above <= r < above + own; every thread tests its own.
  auto seg_of_rank = [&](uint32_t r) {
    for (int sg = tid; sg < NSEG; sg += NTH)
      if (r >= cnt_above(sg) && r < sm.seg_count[sg]) put_seg(sg);
    __syncthreads();
  };
  // First non-empty segment (descending) whose running mass reaches T.
  // Should rounding keep T past the total, the lowest non-empty segment.
  // Picked by a block maximum over a score (hits outrank the rest, the first
  // hit wins), so the answer is unique even where fp64 rounding across
  // thread boundaries makes the prefix dip by an ulp.
  auto seg_of_mass = [&](double T) {
    uint32_t best = 0;
    for (int sg = tid; sg < NSEG; sg += NTH) {
      const uint32_t pos = uint32_t(NSEG - 1 - sg);  // descending position
      if (sm.seg_count[sg] > cnt_above(sg)) {
        const uint32_t score = sm.seg_mass[sg] >= T ? (0x80000000u | (0xFFFFu - pos)) : (pos + 1u);
        best = max(best, score);
      }
    }
    best = block_max_u32<NW>(best, sm);
    const uint32_t pos = (best & 0x80000000u) ? 0xFFFFu - (best & 0xFFFFu) : best - 1u;
    if (tid == 0) put_seg(NSEG - 1 - int(pos));
    __syncthreads();
  };
  // Tokens / mass above segment s (s excluded).
  auto seg_above = [&](int sg) {
    if (tid == 0) put_seg(sg);
    __syncthreads();
  };
  // Inside the segment in bu[0] (above-values in bu[1], bd[0], bd[1]): the key
  // at rank r (mode 0) or where the running mass reaches T (mode 1).  Results:
  // bu[2] = key, bu[3] = tokens above it, bu[4] = its tokens, bd[2] / bd[3] =
  // mass / z-mass above it, bd[4] = its weight.
  auto bin_query = [&](int mode, uint32_t r, double T) {
    fine(int(sm.bu[0]));
    if (w0) {
      const uint32_t s = sm.bu[0];
      const uint32_t key = s * SEGW + uint32_t(SEGW - 1 - lane);
      const uint32_t c = count(key);
      const double d = c ? key_d(key, tau, xmax) : 0.0;
      const double e = c ? exp(d) : 0.0;
      const double m = double(c) * e;
      const double zm = e > 0.0 ? double(c) * e * d : 0.0;
      const uint32_t ci = wave_scan_incl_u32(c);
      const double mi = wave_scan_incl_f64(m), zi = wave_scan_incl_f64(zm);
      const uint32_t cb = sm.bu[1] + ci - c;
      const double mb = sm.bd[0] + (mi - m);
      const double zb = sm.bd[1] + (zi - zm);
      bool hit;
      if (mode == 0) {
        hit = c > 0 && r >= cb && r < cb + c;
      } else {
        hit = c > 0 && sm.bd[0] + mi >= T && (lane == 0 || mb < T);
      }
      const unsigned long long bal = __ballot(hit);
      int src;
      if (bal) {
        src = __ffsll(bal) - 1;
      } else {  // rounding kept the mass target past this segment: its last non-empty key
        const unsigned long long ne = __ballot(c > 0);
        src = ne ? 63 - __clzll(ne) : 0;
      }
      if (lane == src) {
        sm.bu[2] = key;
        sm.bu[3] = cb;
        sm.bu[4] = c;
        sm.bd[2] = mb;
        sm.bd[3] = zb;
        sm.bd[4] = e;
      }
    }
    __syncthreads();
  };

  const uint32_t Vu = uint32_t(a.V);
  // ---- top-k ----
  uint32_t L_k = Vu;
  double Z_k = total_mass;
  if (a.kk > 0 && uint32_t(a.kk) < Vu) {
    L_k = uint32_t(a.kk);
    seg_of_rank(L_k - 1);
    bin_query(0, L_k - 1, 0.0);
    Z_k = sm.bd[2] + double(L_k - sm.bu[3]) * sm.bd[4];
  }
  // ---- inclusive top-p: rank j stays iff the mass before it is < top_p * Z_k ----
  uint32_t L_p = Vu;
  if (a.pf < 1.0f) {
    const double T = double(a.pf) * Z_k;
    seg_of_mass(T);
    bin_query(1, 0, T);
    const double e = sm.bd[4];
    const double room = T - sm.bd[2];
    double n = e > 0.0 ? ceil(room / e) : 1.0;
    n = n < 1.0 ? 1.0 : n;
    L_p = sm.bu[3] + (n >= double(sm.bu[4]) ? sm.bu[4] : uint32_t(n));
    if (L_p > L_k) L_p = L_k;
  }
  // ---- min-p against the row max: the smallest key whose weight reaches min_p ----
  uint32_t L_m = Vu;
  if (a.mpf > 0.0f) {
    if (w0) {
      // the smallest key with z - z_max >= ln(min_p): a 64-way search (each
      // lane tests one key per round, ~3 rounds over 65536 keys), then the
      // boundary is settled with the program's own test exp(z - z_max) >=
      // min_p (keys are in logit order, so both predicates hold on an upper
      // range of keys)
      uint32_t lo = KEY_NEG_INF + 1, hi = kmax;  // the answer is in [lo, hi]; weight(kmax) = 1 >= min_p
      const double mp = double(a.mpf);
      const double lmp = log(mp);
      while (lo < hi) {  // wave-uniform
        const uint32_t step = (hi - lo + 63u) / 64u;
        const uint32_t kl = lo + uint32_t(lane) * step;
        const uint32_t k = kl < hi ? kl : hi;
        const unsigned long long bal = __ballot(key_d(k, tau, xmax) >= lmp);
        if (bal == 0) {
          lo = lo + 63u * step + 1u;  // every tested key fails: the answer lies above lane 63's
        } else {
          const uint32_t f = uint32_t(__ffsll(bal) - 1);
          const uint32_t kf = lo + f * step;
          hi = kf < hi ? kf : hi;
          lo = f == 0 ? lo : lo + (f - 1) * step + 1u;
        }
      }
      if (lane == 0) {
        while (lo > KEY_NEG_INF + 1 && key_weight(lo - 1, tau, xmax) >= mp) --lo;
        while (lo < kmax && key_weight(lo, tau, xmax) < mp) ++lo;
        sm.bu[5] = lo;
      }
    }
    __syncthreads();
    const uint32_t km = sm.bu[5];
    seg_above(int(km / SEGW));
    fine(int(km / SEGW));
    if (w0) {  // tokens of km's segment with key >= km, one key per lane
      const uint32_t k2 = (km / SEGW) * SEGW + uint32_t(lane);
      const uint32_t c = wave_sum_u32(k2 >= km ? count(k2) : 0u);
      if (lane == 0) sm.bu[6] = sm.bu[1] + c;
    }
    __syncthreads();
    L_m = sm.bu[6];
  }
  uint32_t L = L_k < L_p ? L_k : L_p;
  L = L < L_m ? L : L_m;
  if (L < 1) L = 1;

  // ---- the threshold key and the support sums ----
  seg_of_rank(L - 1);
  bin_query(0, L - 1, 0.0);
  const uint32_t K_L = sm.bu[2];
  const uint32_t above_L = sm.bu[3], cnt_L = sm.bu[4];
  const uint32_t r_L = L - above_L;  // tokens of the threshold key inside the support
  const double e_L = sm.bd[4];
  const double d_L = key_d(K_L, tau, xmax);
  const double mass_S = sm.bd[2] + double(r_L) * e_L;
  const double zmass_S = sm.bd[3] + (e_L > 0.0 ? double(r_L) * e_L * d_L : 0.0);

  // ---- target membership (ties at the threshold key resolved by token id) ----
  const uint32_t key_y = a.key_y;
  bool in_s = key_y > K_L;
  if (key_y == K_L) {
    uint32_t below = 0;
    const int yc = int(a.y);
    keys.each([&](uint32_t key, int col) { below += (key == K_L && col < yc) ? 1u : 0u; });
    below = block_sum_u32<NW>(below, sm);
    in_s = below < r_L;
  }

  // ---- dense support ids ----
  uint8_t st = 0;
  if (a.ids_out && a.cap > 0) {
    const typename Keys::Listed listed_data = keys.load_listed();  // in flight during the rank query
    const uint32_t n_out = L < uint32_t(a.cap) ? L : uint32_t(a.cap);
    if (L > uint32_t(a.cap)) st |= kRowTruncated;
    // the key at rank n_out - 1: the support's own threshold query when the
    // whole support fits the cap
    uint32_t K_c = K_L, above_c = above_L, cnt_c = cnt_L;
    if (n_out != L) {
      seg_of_rank(n_out - 1);
      bin_query(0, n_out - 1, 0.0);
      K_c = sm.bu[2];
      above_c = sm.bu[3];
      cnt_c = sm.bu[4];
    }
    const uint32_t r_c = n_out - above_c;
    const bool with_ties = above_c + cnt_c <= uint32_t(Keys::kCollectMax);
    // candidates: every token with key > K_c, plus the tied tokens when they fit
    uint64_t* cand = sm.cand_area();
    if (tid == 0) sm.ncand = 0;
    __syncthreads();
    auto take = [&](uint32_t key, int col) {
      if (key > K_c || (with_ties && key == K_c)) {
        const uint32_t slot = atomicAdd(&sm.ncand, 1u);
        cand[slot] = (uint64_t(key) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(col));
      }
    };
    // the candidates come from the per-thread lists when every thread's list
    // holds all of its tokens with key >= K_c; otherwise from a sweep of the row
    bool listed = false;
    if constexpr (Keys::kTopList) listed = block_max_u32<NW>(keys.listed_from(K_c) ? 0u : 1u, sm) == 0;
    if (listed) {
      keys.each_listed(listed_data, K_c, take);
    } else {
      keys.each(take);
    }
    __syncthreads();
    const uint32_t nc = sm.ncand;
    int64_t* out = a.ids_out + a.row * a.cap;
    const uint32_t n_sorted = with_ties ? n_out : above_c;
    auto id_of = [](uint64_t e) { return int64_t(0xFFFFFFFFu - uint32_t(e & 0xFFFFFFFFu)); };
    if (nc <= uint32_t(NTH)) {
      // rank placement: the candidates are distinct, so each one's position in
      // (key desc, id asc) order is the number of larger ones (the list is
      // read by all threads at once, LDS broadcast, no barriers)
      if (tid < int(nc)) {
        const uint64_t mine = cand[tid];
        uint32_t rank = 0;
        uint32_t j = 0;
        for (; j + 4 <= nc; j += 4)
          rank += uint32_t(cand[j] > mine) + uint32_t(cand[j + 1] > mine) + uint32_t(cand[j + 2] > mine) +
                  uint32_t(cand[j + 3] > mine);
        for (; j < nc; ++j) rank += uint32_t(cand[j] > mine);
        if (rank < n_sorted) out[rank] = id_of(mine);
      }
    } else {
      uint32_t P = 1;
      while (P < nc) P <<= 1;
      for (uint32_t i = nc + tid; i < P; i += NTH) cand[i] = 0;
      __syncthreads();
      // bitonic sort, descending: key descending, token id ascending
      for (uint32_t size = 2; size <= P; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
          for (uint32_t i = tid; i < P; i += NTH) {
            const uint32_t pidx = i ^ stride;
            if (pidx > i) {
              const uint64_t x = cand[i], z = cand[pidx];
              const bool desc = (i & size) == 0;
              if (desc ? (x < z) : (x > z)) {
                cand[i] = z;
                cand[pidx] = x;
              }
            }
          }
          __syncthreads();
        }
      }
      for (uint32_t i = tid; i < n_sorted; i += NTH) out[i] = id_of(cand[i]);
    }
    for (uint32_t i = n_out + tid; i < uint32_t(a.cap); i += NTH) out[i] = -1;
    if (!with_ties) {
      // a very large tie group at K_c: its first r_c tokens in column order, slice by slice
      uint32_t taken = 0;
      keys.opaque();
      for (int j = 0; j < keys.slices(); ++j) {
        uint32_t mine = 0;
        keys.slice(j, [&](uint32_t key, int) { mine += key == K_c ? 1u : 0u; });
        uint32_t tot;
        uint32_t pos = taken + block_excl_scan_u32<NW>(mine, tot, sm);
        keys.slice(j, [&](uint32_t key, int col) {
          if (key == K_c) {
            if (pos < r_c) out[above_c + pos] = col;
            ++pos;
          }
        });
        taken += tot;
      }
    }
  }

  if (tid == 0) {
    const double lms = log(mass_S);
    if (a.entropy) a.entropy[a.row] = float(lms - zmass_S / mass_S);
    if (in_s) {
      a.logprob[a.row] = float(key_d(key_y, tau, xmax) - lms);
    } else {
      a.logprob[a.row] = kNegInf;
      st |= kRowOutside;
    }
    if (a.status) a.status[a.row] = st;
    if (a.support_len) a.support_len[a.row] = int32_t(L);
    if (a.threshold_logit) a.threshold_logit[a.row] = key_logit(K_L);
    if (a.threshold_ties) a.threshold_ties[a.row] = int32_t(r_L);
    if (a.full_lse) a.full_lse[a.row] = float(xmax / tau + log(total_mass));
    if (a.row_max) a.row_max[a.row] = key_logit(kmax);
  }
}

#define VS_ROW_ARGS VS_ROW_ARGS_AT(blockIdx.x)
#define VS_ROW_ARGS_AT(R)                             \
  RowArgs a;                                          \
  a.row = (R);                                        \
  a.V = V;                                            \
  a.tauf = temp ? temp[a.row] : temp_scalar;          \
  a.kk = top_k[a.row];                                \
  a.pf = top_p[a.row];                                \
  a.mpf = min_p[a.row];                               \
  a.y = targets ? targets[a.row] : 0;                 \
  a.rowp = logits + a.row * ld;                       \
  a.logprob = logprob;                                \
  a.entropy = entropy;                                \
  a.status = status;                                  \
  a.support_len = support_len;                        \
  a.threshold_logit = threshold_logit;                \
  a.threshold_ties = threshold_ties;                  \
  a.ids_out = ids_out;                                \
  a.cap = cap;                                        \
  a.full_lse = full_lse;                              \
  a.row_max = row_max;

#define VS_KERNEL_ARGS                                                                                       \
  const uint16_t *__restrict__ logits, int64_t ld, int V, const float *__restrict__ temp, float temp_scalar, \
      const int32_t *__restrict__ top_k, const float *__restrict__ top_p, const float *__restrict__ min_p,   \
      const int64_t *__restrict__ targets, float *__restrict__ logprob, float *__restrict__ entropy,         \
      uint8_t *__restrict__ status, int32_t *__restrict__ support_len, float *__restrict__ threshold_logit,  \
      int32_t *__restrict__ threshold_ties, int64_t *__restrict__ ids_out, int cap,                          \
      float *__restrict__ full_lse, float *__restrict__ row_max, uint8_t *__restrict__ handoff

// Packed-counter path: one counting pass into 65536 16-bit counters.  NV > 0
// keeps the row in registers (NV vectors of 8 tokens per thread); NV == 0
// streams it and re-reads it for the later passes.  A row whose counts would
// overflow 16 bits gets handoff[row] = 1 and nothing else.
template <int NV>
__global__ __launch_bounds__(NV > 0 ? NT : NT_STREAM, 1) void transforms_fast_kernel(VS_KERNEL_ARGS) {
  constexpr int NTH = NV > 0 ? NT : NT_STREAM;
  constexpr int NW = NTH / 64;
  __shared__ Smem sm;
  VS_ROW_ARGS
  const int tid = threadIdx.x;
  if (!params_ok(a)) {
    if (tid == 0) handoff[a.row] = 0;
    write_bad<NTH>(a);
    return;
  }
  a.key_y = key16(a.rowp[a.y]);  // issued now, used after the histogram
  for (int i = tid; i < HALF; i += NTH) sm.hist[i] = 0u;
  __syncthreads();
  using Keys = typename std::conditional<(NV > 0), RegKeys<(NV > 0 ? NV : 1)>, StreamKeys>::type;
  Keys keys;
  uint32_t bad, kmax, n_pad;
  if constexpr (NV > 0) {
    keys.load_count(a.rowp, V, sm.hist, bad, kmax);
    n_pad = uint32_t(NV) * NT * 8u - uint32_t(V);  // padding tokens, all at key 0
  } else {
    keys.rowp = a.rowp;
    keys.V = V;
    keys.rot = 0;
    keys.load_count(sm.hist, kmax);
    n_pad = 0;
  }
  kmax = block_max_u32<NW>(kmax, sm);  // (its barriers also complete the counting)
  if constexpr (NV == 0) {  // (the barriers of the next block maximum publish the merge)
    // NaN and +inf map to keys >= 0xFF80, negative NaNs to keys <= 0x7E (-inf
    // is 0x7F): the row is bad exactly when its largest key or a low bin says so
    bad = (kmax >= 0xFF80u || StreamKeys::low_bad(sm.hist, tid)) ? 1u : 0u;
    if (tid == 0) sm.zero_overflow = StreamKeys::merge_zero(sm.hist) ? 0u : 1u;
  }
  bad = block_max_u32<NW>(bad, sm);
  if (bad || kmax <= KEY_NEG_INF) {  // NaN / +inf present, or every logit is -inf
    if (tid == 0) handoff[a.row] = 0;
    write_bad<NTH>(a);
    return;
  }
  auto count = [&](uint32_t key) -> uint32_t {
    const uint32_t c = (sm.hist[key >> 1] >> ((key & 1u) * 16u)) & 0xFFFFu;
    return key == 0 ? c - n_pad : c;
  };
  const double tau = double(a.tauf);
  const double xmax = double(key_logit(kmax));  // the row maximum (z_max = xmax / tau)
  const uint32_t part = summarize_segments<NTH>(sm.hist, n_pad, tau, xmax, sm);
  // every counter stayed below 2^16 iff the counts add up to the token count
  // (a carry out of a low half, or out of a word, breaks the total); the sum
  // also orders the segment summaries before the queries read them
  if (block_sum_u32<NW>(part, sm) != uint32_t(V) || (NV == 0 && sm.zero_overflow)) {
    if (tid == 0) handoff[a.row] = 1;
    return;
  }
  if (tid == 0) handoff[a.row] = 0;
  finish_row(a, keys, kmax, tau, xmax, sm, [](int) {}, count);
}

// Stream path: the row is re-read from memory for every pass; 32-bit counts.
// With a handoff array, only rows marked 1 are processed.
__global__ __launch_bounds__(NT_STREAM, 1) void transforms_stream_kernel(VS_KERNEL_ARGS) {
  constexpr int NTH = NT_STREAM;
  constexpr int NW = NTH / 64;
  __shared__ Smem sm;
  VS_ROW_ARGS
  if (handoff && handoff[a.row] != 1) return;
  const int tid = threadIdx.x;
  if (!params_ok(a)) {
    write_bad<NTH>(a);
    return;
  }
  a.key_y = key16(a.rowp[a.y]);
  StreamKeys keys{a.rowp, V};
  uint32_t bad = 0, kmax = 0;
  for (int c = tid; c < V; c += NTH) {
    const uint32_t h = a.rowp[c];
    bad |= raw_bad(h) ? 1u : 0u;
    kmax = max(kmax, key16(h));
  }
  kmax = block_max_u32<NW>(kmax, sm);
  bad = block_max_u32<NW>(bad, sm);
  if (bad || kmax <= KEY_NEG_INF) {
    write_bad<NTH>(a);
    return;
  }
  const double tau = double(a.tauf);
  const double xmax = double(key_logit(kmax));  // the row maximum (z_max = xmax / tau)
  for (uint32_t h = 0; h < 2; ++h) {
    for (int i = tid; i < HALF; i += NTH) sm.hist[i] = 0u;
    __syncthreads();
    keys.each([&](uint32_t key, int) {
      if ((key >> 15) == h) atomicAdd(&sm.hist[key & 0x7FFFu], 1u);
    });
    __syncthreads();
    auto count_half = [&](uint32_t key) -> uint32_t { return sm.hist[key & 0x7FFFu]; };
    for (int s = tid; s < NSEG / 2; s += NTH) summarize_segment(int(h) * (NSEG / 2) + s, count_half, tau, xmax, sm);
    __syncthreads();
  }
  if (tid == 0) sm.fine_seg = -1;
  __syncthreads();
  auto fine = [&](int s) {
    if (sm.fine_seg == s) return;
    __syncthreads();
    if (tid < SEGW) sm.fine[tid] = 0u;
    __syncthreads();
    keys.each([&](uint32_t key, int) {
      if ((key >> 6) == uint32_t(s)) atomicAdd(&sm.fine[key & 63u], 1u);
    });
    __syncthreads();
    if (tid == 0) sm.fine_seg = s;
    __syncthreads();
  };
  auto count = [&](uint32_t key) -> uint32_t { return sm.fine[key & 63u]; };
  finish_row(a, keys, kmax, tau, xmax, sm, fine, count);
}

// The count kernel's work on a row after its histogram passed the checks.
__device__ __forceinline__ void count_row_tail(const RowArgs& a, StreamKeys& keys, uint32_t kmax, uint8_t* rec,
                                               uint8_t* handoff, Smem& sm) {
  constexpr int NTH = NT_STREAM;
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x;
  const int V = a.V;
  // Thread t reads segment NSEG-1-t (descending, so the exclusive scan gives
  // the tokens above it), starting at word t % 32 so a wave's reads fall in
  // different banks.
  const int sg = NSEG - 1 - tid;
  const int rot = tid & 31;
  const uint32_t* seg = sm.hist + sg * 32;
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t wd = seg[(i + rot) & 31];
    cnt += (wd & 0xFFFFu) + (wd >> 16);
  }
  uint32_t total, above, entry, n_ne;
  block_excl_scan2_u32<NW>(cnt, cnt ? 1u : 0u, above, entry, total, n_ne, sm);
  // every counter stayed below 2^16 iff the counts add up to the token count;
  // the record holds the count words of at most kRecMaxSegs segments
  if (total != uint32_t(V) || sm.zero_overflow || n_ne > uint32_t(kRecMaxSegs)) {
    if (tid == 0) handoff[a.row] = 1;
    return;
  }
  if (cnt) {  // list entry `entry` (descending segments)
    reinterpret_cast<uint16_t*>(rec + kRecList)[entry] = uint16_t(sg);
    // 16-byte pieces, starting at piece t % 8 (the LDS reads spread over banks)
    const uint4* s4 = reinterpret_cast<const uint4*>(seg);
    uint4* b4 = reinterpret_cast<uint4*>(rec + kRecBlocks) + entry * 8;
#pragma unroll 2
    for (int i = 0; i < 8; ++i) {
      const int c = (i + tid) & 7;
      b4[c] = s4[c];
    }
  }
  uint32_t K_cap = 0;
  uint32_t cand_kind = kCandTokens;
  if (a.ids_out && a.cap > 0) {
    // K_cap, and the largest key any thread dropped from its candidate units,
    // behind one pair of barriers
    const uint32_t r = uint32_t((int64_t(a.cap) < int64_t(V) ? int64_t(a.cap) : int64_t(V)) - 1);
    if (cnt && r >= above && r < above + cnt) {  // exactly one segment holds rank r
      sm.bu[0] = uint32_t(sg);
      sm.bu[1] = above;
    }
    const uint32_t dmax = wave_max_u32(keys.dropped);
    if ((tid & 63) == 0) sm.red_u[tid >> 6] = dmax;
    __syncthreads();
    if (tid < 64) {  // the key inside that segment, one key per lane (descending)
      const uint32_t key = sm.bu[0] * SEGW + uint32_t(SEGW - 1 - tid);
      const uint32_t c = (sm.hist[key >> 1] >> ((key & 1u) * 16u)) & 0xFFFFu;
      const uint32_t cb = sm.bu[1] + wave_scan_incl_u32(c) - c;
      const unsigned long long bal = __ballot(c > 0 && r >= cb && r < cb + c);
      if (tid == __ffsll(bal) - 1) sm.bu[2] = key;
      const uint32_t dm = wave_max_u32(tid < NW ? sm.red_u[tid] : 0u);
      if (tid == 0) sm.bu[3] = dm;
    }
    __syncthreads();
    K_cap = sm.bu[2];
    // Every token with key >= K_cap is in the candidate units reaching K_cap
    // unless some thread dropped such a token: then the row is swept here and
    // the tokens themselves are stored.  Units are stored by position (the
    // finish kernel loads them while it does the segment sums and cuts).
    uint64_t* cg = reinterpret_cast<uint64_t*>(rec + kRecCand);
    cand_kind = sm.bu[3] < K_cap ? kCandUnits : kCandTokens;
    if (cand_kind == kCandUnits) {
      const int nv = keys.nvec();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = keys.vq[i];
        if (q >= 0 && keys.vkey[i] >= K_cap) {
          const uint32_t slot = atomicAdd(&sm.ncand, 1u);
          const uint32_t v1 = q + NTH < nv ? uint32_t(keys.phys(q + NTH, nv)) : 0xFFFFFFFFu;
          if (slot < uint32_t(COLLECT_SPLIT)) cg[slot] = uint64_t(uint32_t(keys.phys(q, nv))) | (uint64_t(v1) << 32);
        }
      }
    } else {
      keys.each([&](uint32_t key, int col) {
        if (key >= K_cap) {
          const uint32_t slot = atomicAdd(&sm.ncand, 1u);
          if (slot < uint32_t(COLLECT_SPLIT)) cg[slot] = (uint64_t(key) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(col));
        }
      });
    }
    __syncthreads();
  }
  if (tid == 0) {
    *reinterpret_cast<uint4*>(rec + kRecHead) = make_uint4(kmax, sm.ncand, K_cap, n_ne);
    reinterpret_cast<uint32_t*>(rec + kRecHead)[4] = cand_kind;
    handoff[a.row] = 2;
  }
}

// The finish kernel's row order: rows whose top-p cut runs without top-k
// (the mass query walks the row's whole prefix) first, then the others, so
// the costlier rows do not end the grid alone.  Two buckets; the order inside
// a bucket is whatever the atomics give (rows are finished independently of
// one another).  Run by the count kernel's first workgroup before its row
// (the finish kernel starts after the whole count kernel).
__device__ __forceinline__ int finish_bucket(int32_t k, float p, int V) { return (k <= 0 || k >= V) && p < 1.0f ? 0 : 1; }
template <int NTH>
__device__ void finish_order(const int32_t* __restrict__ top_k, const float* __restrict__ top_p, int V, int64_t rows,
                             int32_t* __restrict__ order, uint32_t* cnt /* 4 words of LDS */) {
  const int tid = threadIdx.x;
  if (tid < 2) cnt[tid] = 0u;
  __syncthreads();
  for (int64_t r = tid; r < rows; r += NTH) atomicAdd(&cnt[finish_bucket(top_k[r], top_p[r], V)], 1u);
  __syncthreads();
  if (tid == 0) {
    cnt[2] = 0u;
    cnt[3] = cnt[0];
  }
  __syncthreads();
  for (int64_t r = tid; r < rows; r += NTH) order[atomicAdd(&cnt[2 + finish_bucket(top_k[r], top_p[r], V)], 1u)] = int32_t(r);
  __syncthreads();
}

// Split path, first half: one workgroup per row (one thread per segment)
// builds the packed histogram and checks the row as the one-kernel path does,
// then writes the row's record: the count words of every non-empty segment
// (the finish kernel's segment sums and key queries read them), and, for the
// dense ids, every token with key >= K_cap, the key at rank min(cap, V) - 1
// (the dense-id cut lies at or above it), up to COLLECT_SPLIT of them.
// handoff[row]: 0 = done here (bad row), 1 = counter overflow or more than
// kRecMaxSegs non-empty segments (32-bit kernel),
// 2 = the finish kernel completes the row.
__global__ __launch_bounds__(NT_STREAM, 1) void transforms_count_kernel(VS_KERNEL_ARGS,
                                                                       uint8_t *__restrict__ recs,
                                                                       int32_t *__restrict__ order) {
  constexpr int NTH = NT_STREAM;
  constexpr int NW = NTH / 64;
  static_assert(NTH == NSEG, "one thread per segment");
  __shared__ Smem sm;
  if (blockIdx.x == 0) finish_order<NTH>(top_k, top_p, V, int64_t(gridDim.x), order, sm.bu);
  VS_ROW_ARGS
  const int tid = threadIdx.x;
  uint8_t* rec = recs + size_t(a.row) * kRecBytes;
  if (!params_ok(a)) {
    if (tid == 0) handoff[a.row] = 0;
    write_bad<NTH>(a);
    return;
  }
  StreamKeys keys;
  keys.rowp = a.rowp;
  keys.V = V;
  {
    const uint32_t nk = uint32_t(keys.nvec() / 64);  // 1 KiB steps
    keys.rot = nk ? int((uint32_t(a.row) * 2654435761u) % nk) * 64 : 0;
  }
  uint4 first[kInFlight];
  keys.prefetch(first);  // streams while the histogram is cleared
  for (int i = tid; i < HALF / 4; i += NTH) reinterpret_cast<uint4*>(sm.hist)[i] = make_uint4(0, 0, 0, 0);
  if (tid == 0) sm.ncand = 0;
  __syncthreads();
  uint32_t kmax;
  keys.load_count(sm.hist, kmax, first);
  kmax = block_max_u32<NW>(kmax, sm);  // (its barriers also complete the counting)
  uint32_t bad = (kmax >= 0xFF80u || StreamKeys::low_bad(sm.hist, tid)) ? 1u : 0u;
  if (tid == 0) sm.zero_overflow = StreamKeys::merge_zero(sm.hist) ? 0u : 1u;
  bad = block_max_u32<NW>(bad, sm);
  if (bad || kmax <= KEY_NEG_INF) {  // NaN / +inf present, or every logit is -inf
    if (tid == 0) handoff[a.row] = 0;
    write_bad<NTH>(a);
    return;
  }
  count_row_tail(a, keys, kmax, rec, handoff, sm);
}

// Split path, second half: rows marked 2.  The segment summaries come from the
// record's count words (the same sums as the one-kernel path, keys in
// ascending order); a key query loads one segment's words; then everything
// after the histogram exactly as in the one-kernel path.
__global__ __launch_bounds__(NT_FIN, 4) void transforms_finish_kernel(VS_KERNEL_ARGS,
                                                                  const uint8_t *__restrict__ recs,
                                                                  const int32_t *__restrict__ order) {
  constexpr int NTH = NT_FIN;
  __shared__ SmemFin sm;
  VS_ROW_ARGS_AT(int64_t(order[blockIdx.x]))
  if (handoff[a.row] != 2) return;
  const int tid = threadIdx.x;
  const uint8_t* rec = recs + size_t(a.row) * kRecBytes;
  const uint32_t* blocks = reinterpret_cast<const uint32_t*>(rec + kRecBlocks);
  // Everything the row needs first, in one round of loads: the header, the
  // whole segment list, the first FIN_STAGED count blocks and this thread's
  // first candidate (reads past the row's counts stay inside its record).
  const uint4 hd = *reinterpret_cast<const uint4*>(rec + kRecHead);
  const uint32_t cand_kind = reinterpret_cast<const uint32_t*>(rec + kRecHead)[4];
  static_assert(NSEG == 4 * NTH, "four list entries per thread");
  const uint2 lst = reinterpret_cast<const uint2*>(rec + kRecList)[tid];
  constexpr int PER = FIN_STAGED * 8 / NTH;
  uint4 bv[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) bv[u] = reinterpret_cast<const uint4*>(blocks)[tid + u * NTH];
  const uint64_t cand0 = reinterpret_cast<const uint64_t*>(rec + kRecCand)[fin_entry(tid)];
  a.key_y = key16(a.rowp[a.y]);
  // meanwhile: empty summaries and no staging for every segment
  for (int sg = tid; sg < NSEG; sg += NTH) {
    sm.seg_count[sg] = 0u;
    sm.seg_mass[sg] = 0.0;
    sm.seg_zmass[sg] = 0.0;
    sm.seg_slot[sg] = 0xFF;
  }
  const uint32_t kmax = hd.x;
  const uint32_t n_ne = hd.w;
  const uint32_t n_st = min(n_ne, uint32_t(FIN_STAGED));
  const double tau = double(a.tauf);
  const double xmax = double(key_logit(kmax));  // the row maximum (z_max = xmax / tau)
  reinterpret_cast<uint2*>(sm.nelist)[tid] = lst;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const uint32_t idx = uint32_t(tid + u * NTH);
    if (idx < n_st * 8u) reinterpret_cast<uint4*>(sm.blk[idx >> 3])[idx & 7] = bv[u];
  }
  // this thread's first candidate unit: loaded now, used at the dense ids
  uint4 unit0[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  if (cand_kind == kCandUnits && fin_entry(tid) < hd.y) {
    const uint4* pv = reinterpret_cast<const uint4*>(a.rowp);
    const uint32_t v0 = uint32_t(cand0 & 0xFFFFFFFFu), v1 = uint32_t(cand0 >> 32);
    unit0[0] = pv[v0];
    if (v1 != 0xFFFFFFFFu) unit0[1] = pv[v1];
  }
  __syncthreads();
  // Segment summaries, one thread per list entry, with the one-kernel path's
  // arithmetic (staged words read from word e % 32 on: no bank conflicts)
  uint32_t down = 0;  // bit i: this thread's i-th entry needs segment_masses_down
  int i_e = 0;
  for (uint32_t e = uint32_t(tid); e < n_ne; e += NTH, ++i_e) {
    const int sg = sm.nelist[e];
    const int rot = int(e & 31);
    auto sums = [&](auto word) {
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t wd = word((i + rot) & 31);
        cnt += (wd & 0xFFFFu) + (wd >> 16);
      }
      double m = 0.0, zm = 0.0;
      if (sg >= 2 && sg < NSEG - 2 && !segment_masses(sg, word, rot, tau, xmax, m, zm)) down |= 1u << i_e;
      sm.seg_count[sg] = cnt;
      sm.seg_mass[sg] = m;
      sm.seg_zmass[sg] = zm;
    };
    if (e < uint32_t(FIN_STAGED)) {
      sm.seg_slot[sg] = uint8_t(e);
      sums([&](int j) -> uint32_t { return sm.blk[e][j]; });
    } else {
      sums([&](int j) -> uint32_t { return blocks[e * 32 + j]; });
    }
  }
  if (down) {  // rare: segments whose weights leave the normal range
    i_e = 0;
    for (uint32_t e = uint32_t(tid); e < n_ne; e += NTH, ++i_e) {
      if (!((down >> i_e) & 1u)) continue;
      const int sg = sm.nelist[e];
      double m = 0.0, zm = 0.0;
      segment_masses_down(sg, [&](int j) -> uint32_t { return blocks[e * 32 + j]; }, tau, xmax, m, zm);
      sm.seg_mass[sg] = m;
      sm.seg_zmass[sg] = zm;
    }
  }
  if (tid == 0) sm.fine_seg = -1;
  __syncthreads();
  SplitKeys keys;
  keys.rot = 0;
  keys.rowp = a.rowp;
  keys.V = V;
  keys.cand_g = reinterpret_cast<const uint64_t*>(rec + kRecCand);
  keys.cand0 = cand0;
  keys.ncand_g = hd.y;
  keys.kind = cand_kind;
  keys.unit0[0] = unit0[0];
  keys.unit0[1] = unit0[1];
  // a key query's segment: staged words are read in place; others are loaded
  // (list entry e >= FIN_STAGED, found in the descending list)
  auto fine = [&](int s) {
    if (sm.seg_slot[s] != 0xFF || sm.fine_seg == s) return;
    __syncthreads();
    if (tid == 0) sm.bu[7] = 0xFFFFFFFFu;
    __syncthreads();
    for (uint32_t e = uint32_t(FIN_STAGED) + tid; e < n_ne; e += NTH)
      if (sm.nelist[e] == uint16_t(s)) sm.bu[7] = e;
    __syncthreads();
    const uint32_t e = sm.bu[7];
    if (tid < 32) {
      const uint32_t w = e != 0xFFFFFFFFu ? blocks[e * 32 + tid] : 0u;
      sm.fine[2 * tid] = w & 0xFFFFu;
      sm.fine[2 * tid + 1] = w >> 16;
    }
    __syncthreads();
    if (tid == 0) sm.fine_seg = s;
    __syncthreads();
  };
  auto count = [&](uint32_t key) -> uint32_t {
    const uint32_t slot = sm.seg_slot[key >> 6];
    return slot != 0xFFu ? (sm.blk[slot][(key & 63u) >> 1] >> ((key & 1u) * 16u)) & 0xFFFFu : sm.fine[key & 63u];
  };
  finish_row(a, keys, kmax, tau, xmax, sm, fine, count);
}

#undef VS_ROW_ARGS
#undef VS_ROW_ARGS_AT
#undef VS_KERNEL_ARGS


}  // namespace

// Rows longer than the register kernels hold take the split path, whose
// records follow the handoff bytes.
static bool split_rows(int64_t V) { return (V + 7) / 8 > int64_t(20) * NT; }
static size_t handoff_bytes(int64_t rows) { return (size_t(rows) + 255) & ~size_t(255); }
// the finish kernel's row order, after the records
static size_t order_bytes(int64_t rows) { return (size_t(rows) * 4 + 255) & ~size_t(255); }
size_t transforms_workspace_bytes(int64_t rows, int64_t V) {
  return split_rows(V) ? handoff_bytes(rows) + size_t(rows) * kRecBytes + order_bytes(rows) : size_t(rows);
}

int launch_transforms(const uint16_t* logits, int64_t ld, int64_t rows, int64_t V, const float* temp,
                      float temp_scalar, const int32_t* top_k, const float* top_p, const float* min_p,
                      const int64_t* targets, float* logprob, float* entropy, uint8_t* status,
                      int32_t* support_len, float* threshold_logit, int32_t* threshold_ties, int64_t* ids_out,
                      int64_t cap, float* full_lse, float* row_max, uint8_t* handoff, void* stream) {
  if (rows <= 0) return 0;
  if (cap > kTransformsMaxCap) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int vecs = int((V + 7) / 8);
  const int nv = (vecs + NT - 1) / NT;
#define VS_ARGS                                                                                  \
  logits, ld, int(V), temp, temp_scalar, top_k, top_p, min_p, targets, logprob, entropy, status, \
      support_len, threshold_logit, threshold_ties, ids_out, int(cap), full_lse, row_max
  if (nv <= 4) transforms_fast_kernel<4><<<dim3(unsigned(rows)), dim3(NT), 0, s>>>(VS_ARGS, handoff);
  else if (nv <= 10) transforms_fast_kernel<10><<<dim3(unsigned(rows)), dim3(NT), 0, s>>>(VS_ARGS, handoff);
  else if (nv <= 20) transforms_fast_kernel<20><<<dim3(unsigned(rows)), dim3(NT), 0, s>>>(VS_ARGS, handoff);
  else if (!ids_out || cap <= int64_t(COLLECT_SPLIT)) {
    uint8_t* recs = handoff + handoff_bytes(rows);
    int32_t* order = reinterpret_cast<int32_t*>(recs + size_t(rows) * kRecBytes);
    transforms_count_kernel<<<dim3(unsigned(rows)), dim3(NT_STREAM), 0, s>>>(VS_ARGS, handoff, recs, order);
    transforms_finish_kernel<<<dim3(unsigned(rows)), dim3(NT_FIN), 0, s>>>(VS_ARGS, handoff, recs, order);
  } else {
    transforms_fast_kernel<0><<<dim3(unsigned(rows)), dim3(NT_STREAM), 0, s>>>(VS_ARGS, handoff);
  }
  const int rc = int(hipGetLastError());
  if (rc) return rc;
  transforms_stream_kernel<<<dim3(unsigned(rows)), dim3(NT_STREAM), 0, s>>>(VS_ARGS, handoff);
#undef VS_ARGS
  return int(hipGetLastError());
}

}  // namespace vs

// Full-vocabulary scoring over materialised logits, and the fixed-order merge
// of the fused projection's tile partials.
//
// Logits input: one workgroup per row.  Each thread folds a strided share of
// the row (16-byte loads, kRowUnroll of them in flight) into an online
// (max, sum 2^(u-max), sum 2^(u-max)(u-max)) state in registers; the 512
// states are merged by a fixed tree and the row's outputs are written
// directly.  One HBM pass over the logits, no vocabulary-sized temporary and
// no partials (DeepSpec PR #87, Purpose: no vocabulary-sized softmax
// results; xorl issue #71 section 1: the log-sum-exp of the row).
#include "common.h"
#include "launch.h"
#include "../../include/vocabscore.h"

namespace vs {

namespace {

constexpr int kRowThreads = 512;
constexpr int kRowUnroll = 8;
constexpr int kRowBufFlags = 0x00020000;  // dword 3 of a raw buffer resource: 32-bit data format
constexpr int kRowNtAux = 2;              // buffer-load cache policy bit: non-temporal

// Fold n raw logits into the state (base-2 units, u = x * c) against its
// reference m, which moves only when it must: a block whose terms sum to 2^32
// or more (a logit more than 32 above m, the initial m = -inf, or a NaN) is
// folded again after m moves to the block's largest logit, as merge() would.
// The reference then stays within 32 of the running maximum: the entropy sum
// sum 2^d d (d = u - m <= 32) loses about 32 ulps (relative) to cancellation
// when the states are merged, and the common block costs no maximum and no
// rescale.  (A trigger at 2^8 fired in some lane of most waves on N(0, 2)
// logits, and the wave then took the slow path.)  The floor is
// applied only inside the entropy term, so a -inf logit adds exactly 0 and a
// NaN poisons s.
__device__ __forceinline__ void fold_terms(float m, const float* v, int n, float c, float& cs, float& ca) {
  // the first term starts the sums (adding it to zero would change nothing
  // but the sign of a zero entropy term, which no later sum keeps)
  const float d0 = __builtin_fmaf(v[0], c, -m);
  cs = exp2_hw(d0);
  ca = cs * fmaxf(d0, kDFloor);
  for (int i = 1; i < n; ++i) {
    const float d = __builtin_fmaf(v[i], c, -m);
    const float e = exp2_hw(d);
    cs += e;
    ca = __builtin_fmaf(e, fmaxf(d, kDFloor), ca);
  }
}

__device__ __forceinline__ void fold_values(Part& p, const float* v, int n, float c) {
  float cs, ca;
  fold_terms(p.m, v, n, c, cs, ca);
  if (!(cs < 0x1p32f)) {
    float bm = v[0];
    for (int i = 1; i < n; ++i) bm = fmaxf(bm, v[i]);
    const float nm = fmaxf(p.m, bm * c);
    if (nm == kNegInf) {  // only -inf so far, or a NaN that fmaxf dropped
      for (int i = 0; i < n; ++i)
        if (v[i] != v[i]) p.s = __builtin_nanf("");
      return;
    }
    if (nm > p.m) {
      if (!(p.m == kNegInf && p.s == 0.0f)) {
        const float d = p.m - nm;
        const float f = exp2_hw(d);
        p.a = f == 0.0f ? 0.0f : f * __builtin_fmaf(p.s, d, p.a);  // (p.s * d may overflow when f = 0)
        p.s *= f;
      }
      p.m = nm;
    }
    fold_terms(p.m, v, n, c, cs, ca);
  }
  p.s += cs;
  p.a += ca;
}

template <int DT>
__device__ __forceinline__ void unpack(const uint4& w, float* v) {
  v[0] = bf16_lo(w.x);
  v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y);
  v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z);
  v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w);
  v[7] = bf16_hi(w.w);
}

// This thread's share of one row: vectors q = tid, tid + NT, ... then a scalar tail.
template <int DT>
__device__ __forceinline__ Part row_state(const void* rowp, int64_t V, float c) {
  constexpr int VEC = DT == VS_BF16 ? 8 : 4;
  Part p{kNegInf, 0.0f, 0.0f};
  const int tid = threadIdx.x;
  const bool aligned = (reinterpret_cast<uintptr_t>(rowp) & 15) == 0;
  const int64_t nvec = aligned ? V / VEC : 0;
  int64_t q = tid;
  float v[VEC];
  if (DT == VS_BF16) {
    // A ring of kRowUnroll buffer loads: chunk k's slot is unpacked, refilled
    // with chunk k + kRowUnroll, then folded, so the loads stay in flight
    // while the thread folds and no register is copied.  The ring covers the
    // nu chunks every thread has (a uniform count, so a chunk's offset is a
    // scalar operand and costs no vector instruction); a thread's one extra
    // chunk comes last.  Chunks are folded in ascending order, as a plain loop
    // would fold them.
    const int64_t nu = nvec / kRowThreads;
    constexpr int U = kRowUnroll;
    if (nu >= U) {
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(rowp), (short)0, int(nvec * 16), kRowBufFlags);
      const uint32_t vo = uint32_t(tid) * 16u;
      auto chunk = [&](int64_t k) -> uint4 {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, uint32_t(k) * uint32_t(kRowThreads * 16),
                                                              kRowNtAux);
        return make_uint4(x.x, x.y, x.z, x.w);
      };
      uint4 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = chunk(u);
      int64_t i = 0;
      for (; i + 2 * U <= nu; i += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          unpack<DT>(w[u], v);
          w[u] = chunk(i + U + u);
          fold_values(p, v, VEC, c);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {  // chunks i .. i+U-1; refills only below nu
        unpack<DT>(w[u], v);
        if (i + U + u < nu) w[u] = chunk(i + U + u);
        fold_values(p, v, VEC, c);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)  // the last nu - i - U < U chunks
        if (i + U + u < nu) {
          unpack<DT>(w[u], v);
          fold_values(p, v, VEC, c);
        }
      if (tid + nu * kRowThreads < nvec) {  // this thread's extra chunk
        unpack<DT>(chunk(nu), v);
        fold_values(p, v, VEC, c);
      }
    } else {
      const uint4* pv = static_cast<const uint4*>(rowp) + tid;
      const int64_t n = nvec > tid ? (nvec - 1 - tid) / kRowThreads + 1 : 0;  // this thread's chunks
      for (int64_t k = 0; k < n; ++k) {
        unpack<DT>(stream_load(pv + k * kRowThreads), v);
        fold_values(p, v, VEC, c);
      }
    }
    for (int64_t i = nvec * VEC + tid; i < V; i += kRowThreads) {
      v[0] = bf16_to_f32(static_cast<const uint16_t*>(rowp)[i]);
      fold_values(p, v, 1, c);
    }
  } else {
    const float4* pv = static_cast<const float4*>(rowp);
    for (; q + int64_t(kRowUnroll - 1) * kRowThreads < nvec; q += int64_t(kRowUnroll) * kRowThreads) {
      float4 w[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) w[u] = stream_load(pv + q + u * kRowThreads);
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        v[0] = w[u].x;
        v[1] = w[u].y;
        v[2] = w[u].z;
        v[3] = w[u].w;
        fold_values(p, v, VEC, c);
      }
    }
    for (; q < nvec; q += kRowThreads) {
      const float4 w = stream_load(pv + q);
      v[0] = w.x;
      v[1] = w.y;
      v[2] = w.z;
      v[3] = w.w;
      fold_values(p, v, VEC, c);
    }
    for (int64_t i = nvec * VEC + tid; i < V; i += kRowThreads) {
      v[0] = static_cast<const float*>(rowp)[i];
      fold_values(p, v, 1, c);
    }
  }
  return p;
}

// Row outputs from the row's merged base-2 state (shared by both input kinds).
__device__ __forceinline__ void write_row(Part acc, int64_t row, float c, bool tau_valid, int64_t y, int64_t V,
                                          float zy_raw, bool have_zy, float* lse, float* logprob, float* entropy,
                                          uint8_t* status, int mode) {
  const bool ok_in = tau_valid && y >= 0 && y < V;
  const float l2s = log2_hw(acc.s);
  const float lse2 = acc.m + l2s;  // base-2 LSE
  const bool ok = ok_in && (lse2 > -__builtin_inff()) && (lse2 < __builtin_inff()) && have_zy;
  const float zy = ok ? zy_raw * c : 0.0f;
  const float nan = __builtin_nanf("");
  // (u_y - m) - log2 s: forming u_y - (m + log2 s) would drop log2 s below
  // one ulp of m at large magnitudes
  const float lp = ok ? kLn2 * ((zy - acc.m) - l2s) : nan;
  if (mode == kMergeFull) {
    if (lse) lse[row] = ok ? kLn2 * lse2 : nan;
    logprob[row] = lp;
    if (entropy) entropy[row] = ok ? kLn2 * (l2s - acc.a / acc.s) : nan;
    if (status) status[row] = ok ? 0 : kRowBad;
  } else {
    logprob[row] = lp;
    if (entropy) entropy[row] = ok ? 0.0f : nan;
    if (status) status[row] = ok ? (kRowEmpty | kRowFallback) : kRowBad;
  }
}

template <int DT>
__global__ __launch_bounds__(kRowThreads) void logits_row_kernel(
    const void* __restrict__ logits, int64_t ld, int64_t V, const float* __restrict__ temp, float temp_scalar,
    const int32_t* __restrict__ row_map, const int32_t* __restrict__ row_count, const int64_t* __restrict__ targets,
    float* __restrict__ lse, float* __restrict__ logprob, float* __restrict__ entropy, uint8_t* __restrict__ status,
    int mode) {
  constexpr int ES = DT == VS_BF16 ? 2 : 4;
  constexpr int NW = kRowThreads / 64;
  const int64_t slot = blockIdx.x;
  if (row_count && slot >= *row_count) return;
  const int64_t row = row_map ? int64_t(row_map[slot]) : slot;
  const float tau = temp ? temp[row] : temp_scalar;
  const float c = DT == VS_BF16 ? scale16(kLog2e / tau) : kLog2e / tau;
  const char* rowp = static_cast<const char*>(logits) + row * ld * ES;
  Part p = row_state<DT>(rowp, V, c);
  // fixed tree: inside each wave, then the wave states in order
  __shared__ float red[NW][3];
  p = wave_merge_to_lane0(p);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[w][0] = p.m;
    red[w][1] = p.s;
    red[w][2] = p.a;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  Part acc = Part{red[0][0], red[0][1], red[0][2]};
#pragma unroll
  for (int i = 1; i < NW; ++i) acc = merge(acc, Part{red[i][0], red[i][1], red[i][2]});
  const int64_t y = targets[row];
  const bool yv = y >= 0 && y < V;
  const float zraw = yv ? (DT == VS_BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(rowp)[y])
                                         : reinterpret_cast<const float*>(rowp)[y])
                        : 0.0f;
  write_row(acc, row, c, tau_ok(tau), y, V, zraw, true, lse, logprob, entropy, status, mode);
}

// ---------------------------------------------------------------------------
// Fixed-order merge: one wave per row.  Lane l owns a contiguous run of
// vocab_chunk-wide chunks; inside a chunk tiles are merged in ascending
// order, chunk states are merged in ascending order inside the lane, and the
// 64 lane states by a fixed tree.  Then the row outputs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(const float4* __restrict__ partials, int n_tiles, int tpc,
                                                    int64_t rows, const int32_t* __restrict__ row_map,
                                                    const int32_t* __restrict__ row_count,
                                                    const float* __restrict__ temp, float temp_scalar,
                                                    const int64_t* __restrict__ targets, int64_t V, LogitsArg lg,
                                                    const float* __restrict__ zy_raw, float* __restrict__ lse,
                                                    float* __restrict__ logprob, float* __restrict__ entropy,
                                                    uint8_t* __restrict__ status, int mode) {
  const int64_t slot = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (slot >= rows) return;
  if (row_count && slot >= *row_count) return;
  const int lane = threadIdx.x & 63;
  const int64_t row = row_map ? int64_t(row_map[slot]) : slot;
  const float tau = temp ? temp[row] : temp_scalar;
  const float c = kLog2e / tau;

  const int n_chunks = (n_tiles + tpc - 1) / tpc;
  const int cpl = (n_chunks + 63) / 64;
  Part acc{kNegInf, 0.0f, 0.0f};
  const float4* pr = partials + slot * n_tiles;
  for (int ch = lane * cpl; ch < (lane + 1) * cpl && ch < n_chunks; ++ch) {
    Part cs{kNegInf, 0.0f, 0.0f};
    const int t1 = (ch + 1) * tpc < n_tiles ? (ch + 1) * tpc : n_tiles;
    for (int t = ch * tpc; t < t1; ++t) {
      float4 q = pr[t];
      cs = merge(cs, Part{q.x, q.y, q.z});
    }
    acc = merge(acc, cs);
  }
  acc = wave_merge_to_lane0(acc);
  if (lane != 0) return;

  const int64_t y = targets[row];
  const bool yv = y >= 0 && y < V;
  float zraw = 0.0f;
  if (yv) {
    if (zy_raw) {
      zraw = zy_raw[slot];
    } else if (lg.dtype == VS_BF16) {
      zraw = bf16_to_f32(static_cast<const uint16_t*>(lg.ptr)[row * lg.ld + y]);
    } else {
      zraw = static_cast<const float*>(lg.ptr)[row * lg.ld + y];
    }
  }
  write_row(acc, row, c, tau_ok(tau), y, V, zraw, true, lse, logprob, entropy, status, mode);
}

__global__ void zero_i32_kernel(int32_t* p, int64_t n) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

int launch_logits_rows(LogitsArg lg, int64_t rows, int64_t V, const float* temp, float temp_scalar,
                       const int32_t* row_map, const int32_t* row_count, const int64_t* targets, float* lse,
                       float* logprob, float* entropy, uint8_t* status, int mode, void* stream) {
  if (rows <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (lg.dtype == VS_BF16) {
    logits_row_kernel<VS_BF16><<<dim3(unsigned(rows)), dim3(kRowThreads), 0, s>>>(
        lg.ptr, lg.ld, V, temp, temp_scalar, row_map, row_count, targets, lse, logprob, entropy, status, mode);
  } else {
    logits_row_kernel<VS_F32><<<dim3(unsigned(rows)), dim3(kRowThreads), 0, s>>>(
        lg.ptr, lg.ld, V, temp, temp_scalar, row_map, row_count, targets, lse, logprob, entropy, status, mode);
  }
  return int(hipGetLastError());
}

int launch_merge(const void* partials, int n_tiles, int tiles_per_chunk, int64_t rows, const int32_t* row_map,
                 const int32_t* row_count, const float* temp, float temp_scalar, const int64_t* targets, int64_t V,
                 LogitsArg lg, const float* zy_raw, float* lse, float* logprob, float* entropy, uint8_t* status,
                 int mode, void* stream) {
  if (rows <= 0) return 0;
  const int64_t blocks = (rows + 3) / 4;
  merge_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const float4*>(partials), n_tiles, tiles_per_chunk, rows, row_map, row_count, temp, temp_scalar,
      targets, V, lg, zy_raw, lse, logprob, entropy, status, mode);
  return int(hipGetLastError());
}

int launch_zero_i32(int32_t* p, int64_t n, void* stream) {
  if (n <= 0) return 0;
  zero_i32_kernel<<<dim3(unsigned((n + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(p, n);
  return int(hipGetLastError());
}

}  // namespace vs

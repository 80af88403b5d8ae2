// Full-vocabulary scoring over materialised logits, and the fixed-order merge
// shared with the fused projection.
//
// Logits-input sweep: one workgroup per (row, 8192-column tile), 16-byte
// coalesced loads, each thread folds its 32 columns into an online state in
// registers, the workgroup merges its 256 states with a fixed tree and writes
// one partial.  One HBM pass over the logits; no vocabulary-sized temporary
// (DeepSpec PR #87, Purpose: the vocabulary-sized FP32 softmax results are
// what the page removes; xorl issue #71 section 1: chunked LSE).
#include "common.h"
#include "launch.h"
#include "../../include/vocabscore.h"

namespace vs {

namespace {

constexpr int kThreads3 = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load: the logits are read exactly once.
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 stream_load(const float4* p) {
  f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
constexpr int kPerThread3 = kLogitsTile / kThreads3;  // 32 columns per thread

// One row tile of bf16 logits.  Vector path when the row base is 16-byte aligned.
__device__ __forceinline__ Part tile_state_bf16(const uint16_t* row, int64_t c0, int64_t c1, float c) {
  float vals[kPerThread3];
  const int tid = threadIdx.x;
  const bool aligned = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  if (aligned && c1 - c0 == kLogitsTile) {
    const uint4* p = reinterpret_cast<const uint4*>(row + c0);
#pragma unroll
    for (int j = 0; j < kPerThread3 / 8; ++j) {
      uint4 w = stream_load(p + j * kThreads3 + tid);
      vals[8 * j + 0] = bf16_lo(w.x);
      vals[8 * j + 1] = bf16_hi(w.x);
      vals[8 * j + 2] = bf16_lo(w.y);
      vals[8 * j + 3] = bf16_hi(w.y);
      vals[8 * j + 4] = bf16_lo(w.z);
      vals[8 * j + 5] = bf16_hi(w.z);
      vals[8 * j + 6] = bf16_lo(w.w);
      vals[8 * j + 7] = bf16_hi(w.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread3 / 8; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int64_t col = c0 + int64_t(j * kThreads3 + tid) * 8 + e;
        vals[8 * j + e] = col < c1 ? bf16_to_f32(row[col]) : kNegInf;
      }
    }
  }
  float mx = vals[0];
#pragma unroll
  for (int i = 1; i < kPerThread3; ++i) mx = fmaxf(mx, vals[i]);
  Part p;
  p.m = mx * c;
  p.s = 0.0f;
  p.a = 0.0f;
  if (mx == kNegInf) {
    p.s = empty_block_s<kPerThread3>(vals);
    return p;
  }
#pragma unroll
  for (int i = 0; i < kPerThread3; ++i) fold(__builtin_fmaf(vals[i], c, -p.m), p.s, p.a);
  return p;
}

__device__ __forceinline__ Part tile_state_f32(const float* row, int64_t c0, int64_t c1, float c) {
  float vals[kPerThread3];
  const int tid = threadIdx.x;
  const bool aligned = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  if (aligned && c1 - c0 == kLogitsTile) {
    const float4* p = reinterpret_cast<const float4*>(row + c0);
#pragma unroll
    for (int j = 0; j < kPerThread3 / 4; ++j) {
      float4 w = stream_load(p + j * kThreads3 + tid);
      vals[4 * j + 0] = w.x;
      vals[4 * j + 1] = w.y;
      vals[4 * j + 2] = w.z;
      vals[4 * j + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread3 / 4; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int64_t col = c0 + int64_t(j * kThreads3 + tid) * 4 + e;
        vals[4 * j + e] = col < c1 ? row[col] : kNegInf;
      }
    }
  }
  float mx = vals[0];
#pragma unroll
  for (int i = 1; i < kPerThread3; ++i) mx = fmaxf(mx, vals[i]);
  Part p;
  p.m = mx * c;
  p.s = 0.0f;
  p.a = 0.0f;
  if (mx == kNegInf) {
    p.s = empty_block_s<kPerThread3>(vals);
    return p;
  }
#pragma unroll
  for (int i = 0; i < kPerThread3; ++i) fold(__builtin_fmaf(vals[i], c, -p.m), p.s, p.a);
  return p;
}

// Workgroup merge of the 4 wave states (fixed order), result in thread 0.
__device__ __forceinline__ Part block_merge_256(Part p) {
  __shared__ float sm[4][3];
  p = wave_merge_to_lane0(p);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[w][0] = p.m;
    sm[w][1] = p.s;
    sm[w][2] = p.a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    Part q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = Part{sm[i][0], sm[i][1], sm[i][2]};
    p = merge(merge(q[0], q[1]), merge(q[2], q[3]));
  }
  return p;
}

template <int DT>
__global__ __launch_bounds__(kThreads3) void logits_partials_kernel(const void* __restrict__ logits, int64_t ld,
                                                                    int64_t V, int n_tiles,
                                                                    const float* __restrict__ temp, float temp_scalar,
                                                                    const int32_t* __restrict__ row_map,
                                                                    const int32_t* __restrict__ row_count,
                                                                    float4* __restrict__ partials) {
  const int64_t slot = int64_t(blockIdx.x) / n_tiles;
  const int tile = int(int64_t(blockIdx.x) - slot * n_tiles);
  if (row_count && slot >= *row_count) return;
  const int64_t row = row_map ? int64_t(row_map[slot]) : slot;
  const float tau = temp ? temp[row] : temp_scalar;
  const float c = kLog2e / tau;
  const int64_t c0 = int64_t(tile) * kLogitsTile;
  const int64_t c1 = c0 + kLogitsTile < V ? c0 + kLogitsTile : V;
  Part p;
  if (DT == VS_BF16) {
    p = tile_state_bf16(static_cast<const uint16_t*>(logits) + row * ld, c0, c1, c);
  } else {
    p = tile_state_f32(static_cast<const float*>(logits) + row * ld, c0, c1, c);
  }
  p = block_merge_256(p);
  if (threadIdx.x == 0) partials[slot * n_tiles + tile] = make_float4(p.m, p.s, p.a, 0.0f);
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
  const bool ok_in = tau_ok(tau) && y >= 0 && y < V;
  const float l2s = log2_hw(acc.s);
  const float lse2 = acc.m + l2s;  // base-2 LSE
  const bool ok = ok_in && (lse2 > -__builtin_inff()) && (lse2 < __builtin_inff());
  float zy = 0.0f;
  if (ok) {
    if (zy_raw) {
      zy = zy_raw[slot] * c;
    } else if (lg.dtype == VS_BF16) {
      zy = bf16_to_f32(static_cast<const uint16_t*>(lg.ptr)[row * lg.ld + y]) * c;
    } else {
      zy = static_cast<const float*>(lg.ptr)[row * lg.ld + y] * c;
    }
  }
  const float nan = __builtin_nanf("");
  const float lp = ok ? kLn2 * (zy - lse2) : nan;
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

__global__ void zero_i32_kernel(int32_t* p, int64_t n) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

int launch_logits_partials(LogitsArg lg, int64_t rows, int64_t V, const float* temp, float temp_scalar,
                           const int32_t* row_map, const int32_t* row_count, void* partials, void* stream) {
  const int n_tiles = int((V + kLogitsTile - 1) / kLogitsTile);
  const int64_t blocks = rows * n_tiles;
  if (blocks <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (lg.dtype == VS_BF16) {
    logits_partials_kernel<VS_BF16><<<dim3(unsigned(blocks)), dim3(kThreads3), 0, s>>>(
        lg.ptr, lg.ld, V, n_tiles, temp, temp_scalar, row_map, row_count, static_cast<float4*>(partials));
  } else {
    logits_partials_kernel<VS_F32><<<dim3(unsigned(blocks)), dim3(kThreads3), 0, s>>>(
        lg.ptr, lg.ld, V, n_tiles, temp, temp_scalar, row_map, row_count, static_cast<float4*>(partials));
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

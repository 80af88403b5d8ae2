// Recorded-support scoring (SkyRL PR #2004: replay logprob and entropy
// renormalised over the sampler's recorded support, dense padded ids).
//
// One workgroup per token row:
//   1. the row's ids go to LDS; ids >= V and repeated ids are detected
//      (the row becomes BAD_INPUT and no weight row is read for it);
//   2. the support logits are gathered: logits[t, id] for a logits source,
//      or dot(bf16(hidden[t]), W[id]) for a hidden/weight source, with the
//      hidden row staged once in LDS and every selected weight row streamed
//      by one wave with 16-byte coalesced loads (the page's review asks for
//      exactly this: chunk by token rows, never gather the hidden tensor per
//      pair);
//   3. wave 0 folds the support into (max, sum-exp, sum p*z) and writes the
//      row's logprob, entropy and status.  A one-id support gives exactly 0
//      and 0: its only term has d = u - max = 0, 2^0 = 1, 0 * 1 = 0.
// Empty rows flagged as synthetic EOS are appended to a list that the host
// then sends through the full-vocabulary sweep.
#include "common.h"
#include "launch.h"
#include "../../include/vocabscore.h"

namespace vs {

namespace {

constexpr int NT = 256;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + dot(8 bf16 of w, 8 bf16 of h), fp32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot8(uint4 w, uint4 h, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, h.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, h.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, h.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, h.w), acc, false);
  return acc;
}

template <bool FUSED>
__global__ __launch_bounds__(NT) void support_kernel(
    const void* __restrict__ src, int src_dtype, int64_t ld_src, const uint16_t* __restrict__ weight, int64_t ld_w,
    int64_t H, int64_t V, const float* __restrict__ temp, float temp_scalar, const int64_t* __restrict__ ids,
    int width, int64_t ld_ids, const int64_t* __restrict__ targets, const uint8_t* __restrict__ fallback,
    float* __restrict__ logprob, float* __restrict__ entropy, uint8_t* __restrict__ status,
    int32_t* __restrict__ fb_list, int32_t* __restrict__ fb_count, const int32_t* __restrict__ order) {
  // No contraction in this kernel: u = x * c is rounded before u - max, so
  // the maximum's own term is exactly 2^0 = 1 with d = 0.
#pragma clang fp contract(off)
  // dynamic LDS, sized by the launch: the hidden row as bf16 (H/8 chunks,
  // fused source only), then the row's ids and their logits.  Sizing the id
  // arrays by the width instead of its maximum keeps a 64-wide support at
  // 15 KiB per workgroup at H = 7168, so eight workgroups share a CU.
  extern __shared__ uint4 dyn[];
  uint4* hs = dyn;
  int64_t* sid = reinterpret_cast<int64_t*>(dyn + (FUSED ? H / 8 : 0));
  float* sx = reinterpret_cast<float*>(sid + width);
  __shared__ int s_bad, s_count;

  const int64_t row = order ? int64_t(order[blockIdx.x]) : int64_t(blockIdx.x);
  const int tid = threadIdx.x;
  const float tau = temp ? temp[row] : temp_scalar;
  if (tid == 0) {
    s_bad = tau_ok(tau) ? 0 : 1;
    s_count = 0;
  }
  __syncthreads();
  int my_count = 0;
  for (int j = tid; j < width; j += NT) {
    const int64_t id = ids[row * ld_ids + j];
    sid[j] = id;
    if (id >= V) atomicOr(&s_bad, 1);
    if (id >= 0) ++my_count;
  }
  if (my_count) atomicAdd(&s_count, my_count);
  __syncthreads();
  // repeated ids: compare each id with the ids before it
  for (int j = tid; j < width; j += NT) {
    const int64_t id = sid[j];
    if (id < 0) continue;
    for (int k = 0; k < j; ++k)
      if (sid[k] == id) {
        atomicOr(&s_bad, 1);
        break;
      }
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  const int count = s_count;
  const float nan = __builtin_nanf("");

  if (bad) {
    if (tid == 0) {
      logprob[row] = nan;
      if (entropy) entropy[row] = nan;
      if (status) status[row] = kRowBad;
    }
    return;
  }
  if (count == 0) {
    if (tid == 0) {
      if (fallback && fallback[row]) {
        fb_list[atomicAdd(fb_count, 1)] = int32_t(row);  // outputs written by the fallback sweep
      } else {
        logprob[row] = 0.0f;
        if (entropy) entropy[row] = 0.0f;
        if (status) status[row] = kRowEmpty;
      }
    }
    return;
  }

  // ---- gather the support logits (raw x, before temperature) ----
  if (FUSED) {
    const int64_t nch = H / 8;
    if (src_dtype == VS_BF16) {
      const uint4* hrow = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + row * ld_src);
      for (int64_t q = tid; q < nch; q += NT) hs[q] = hrow[q];
    } else {
      const float4* hrow = reinterpret_cast<const float4*>(static_cast<const float*>(src) + row * ld_src);
      for (int64_t q = tid; q < nch; q += NT) {
        float4 lo = hrow[2 * q], hi = hrow[2 * q + 1];
        float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t u = __float_as_uint(f[e]);
          b[e] = ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : ((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
        }
        hs[q] = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
      }
    }
    __syncthreads();
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int j = wave; j < width; j += NT / 64) {
      const int64_t id = sid[j];
      if (id < 0) continue;
      const uint4* wrow = reinterpret_cast<const uint4*>(weight + id * ld_w);
      float acc0 = 0.0f, acc1 = 0.0f;
      int64_t q = lane;
      for (; q + 64 < nch; q += 128) {
        const uint4 w0 = stream_load(wrow + q), w1 = stream_load(wrow + q + 64);
        acc0 = dot8(w0, hs[q], acc0);
        acc1 = dot8(w1, hs[q + 64], acc1);
      }
      for (; q < nch; q += 64) acc0 = dot8(stream_load(wrow + q), hs[q], acc0);
      float acc = acc0 + acc1;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc += shfl_xor_f(acc, off);
      if (lane == 0) sx[j] = acc;
    }
  } else {
    for (int j = tid; j < width; j += NT) {
      const int64_t id = sid[j];
      if (id < 0) continue;
      sx[j] = src_dtype == VS_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(src)[row * ld_src + id])
                                   : static_cast<const float*>(src)[row * ld_src + id];
    }
  }
  __syncthreads();
  if (tid >= 64) return;

  // ---- wave 0: fold the support ----
  const int lane = tid;
  const float c = kLog2e / tau;
  const int64_t y = targets[row];
  float mx = kNegInf;
  float uy = 0.0f;
  int found = 0;
  for (int j = lane; j < width; j += 64) {
    if (sid[j] < 0) continue;
    const float u = sx[j] * c;
    mx = fmaxf(mx, u);
    if (sid[j] == y) {
      uy = u;
      found = 1;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
  Part p{mx, 0.0f, 0.0f};
  if (mx != kNegInf) {
    for (int j = lane; j < width; j += 64) {
      if (sid[j] < 0) continue;
      fold(sx[j] * c - mx, p.s, p.a);
    }
  }
  p = wave_merge_to_lane0(p);
  // the lane that saw the target publishes it
  const unsigned long long who = __ballot(found);
  const int src_lane = who ? __ffsll(who) - 1 : 0;
  uy = __shfl(uy, src_lane, 64);
  if (lane != 0) return;
  const float l2s = log2_hw(p.s);
  const float lse2 = p.m + l2s;
  const bool ok = (y >= 0) && (y < V) && (lse2 > -__builtin_inff()) && (lse2 < __builtin_inff());
  if (!ok) {
    logprob[row] = nan;
    if (entropy) entropy[row] = nan;
    if (status) status[row] = kRowBad;
    return;
  }
  if (entropy) entropy[row] = kLn2 * (l2s - p.a / p.s);
  if (who) {
    logprob[row] = kLn2 * ((uy - p.m) - l2s);
    if (status) status[row] = 0;
  } else {
    logprob[row] = kNegInf;
    if (status) status[row] = kRowOutside;
  }
}

// Workgroup order of the hidden/weight source.  A row costs in proportion to
// its number of ids, and the workgroups of one launch all run at once, eight
// to a CU, workgroup b on CU b mod (CU count) when the grid is dealt out in
// order; a CU then finishes with its heaviest share.  The rows are ranked by
// their id count (descending) and rank r = m * G + j (G = CU count) goes to
// workgroup m * G + j for even m and m * G + G - 1 - j for odd m, so each CU
// gets ranks j, 2G - 1 - j, 2G + j, ...: near-equal shares.  A last partial
// group keeps rank order.  The outputs do not depend on the order.
constexpr int kWidthThreads = 256;
__global__ __launch_bounds__(kWidthThreads) void support_width_kernel(const int64_t* __restrict__ ids, int width,
                                                                     int64_t ld_ids, int64_t rows,
                                                                     int32_t* __restrict__ count) {
  const int64_t row = int64_t(blockIdx.x) * (kWidthThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (int j = lane; j < width; j += 64) n += ids[row * ld_ids + j] >= 0 ? 1 : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) n += __shfl_xor(n, off, 64);
  if (lane == 0) count[row] = n;
}
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void support_order_kernel(const int32_t* __restrict__ count, int width,
                                                                     int64_t rows, int G, int32_t* __restrict__ order) {
  extern __shared__ uint32_t bucket[];  // width + 1 counters, then their starts
  const int tid = threadIdx.x;
  for (int w = tid; w <= width; w += kOrderThreads) bucket[w] = 0u;
  __syncthreads();
  for (int64_t r = tid; r < rows; r += kOrderThreads) atomicAdd(&bucket[count[r]], 1u);
  __syncthreads();
  if (tid == 0) {  // starts in descending width
    uint32_t b = 0;
    for (int w = width; w >= 0; --w) {
      const uint32_t c = bucket[w];
      bucket[w] = b;
      b += c;
    }
  }
  __syncthreads();
  const int64_t full = rows / G * G;
  for (int64_t r = tid; r < rows; r += kOrderThreads) {
    const int64_t rank = int64_t(atomicAdd(&bucket[count[r]], 1u));
    const int64_t m = rank / G, j = rank - m * G;
    const int64_t b = rank >= full ? rank : m * G + ((m & 1) ? G - 1 - j : j);
    order[b] = int32_t(r);
  }
}

// dynamic LDS of one workgroup: [bf16 hidden row][ids int64][logits fp32]
size_t support_lds_bytes(bool fused, int64_t H, int64_t width) {
  return (fused ? size_t(H / 8) * 16 : 0) + size_t(width) * 8 + size_t(width) * 4;
}

}  // namespace

const int32_t* support_row_order(const int64_t* ids, int64_t width, int64_t ld_ids, int64_t rows, int32_t* ws,
                                 void* stream) {
  int ncu = 0;
  if (width <= 1 || device_cu_count(&ncu) != 0 || rows < 2 * int64_t(ncu)) return nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* count = ws + rows;  // [rows] id counts after the [rows] order
  support_width_kernel<<<dim3(unsigned((rows + 3) / 4)), dim3(kWidthThreads), 0, s>>>(ids, int(width), ld_ids, rows,
                                                                                      count);
  support_order_kernel<<<dim3(1), dim3(kOrderThreads), size_t(width + 1) * 4, s>>>(count, int(width), rows, ncu, ws);
  return hipGetLastError() == hipSuccess ? ws : nullptr;
}

int launch_support_logits(LogitsArg lg, int64_t rows, int64_t V, const float* temp, float temp_scalar,
                          const int64_t* ids, int64_t width, int64_t ld_ids, const int64_t* targets,
                          const uint8_t* fallback, float* logprob, float* entropy, uint8_t* status,
                          int32_t* fb_list, int32_t* fb_count, void* stream) {
  if (rows <= 0) return 0;
  const size_t lds = support_lds_bytes(false, 0, width);
  support_kernel<false><<<dim3(unsigned(rows)), dim3(NT), lds, static_cast<hipStream_t>(stream)>>>(
      lg.ptr, lg.dtype, lg.ld, nullptr, 0, 0, V, temp, temp_scalar, ids, int(width), ld_ids, targets, fallback,
      logprob, entropy, status, fb_list, fb_count, nullptr);
  return int(hipGetLastError());
}

int launch_support_fused(const void* hidden, int hidden_dtype, int64_t ld_hidden, const uint16_t* weight,
                         int64_t ld_weight, int64_t rows, int64_t H, int64_t V, const float* temp,
                         float temp_scalar, const int64_t* ids, int64_t width, int64_t ld_ids,
                         const int64_t* targets, const uint8_t* fallback, float* logprob, float* entropy,
                         uint8_t* status, int32_t* fb_list, int32_t* fb_count, int32_t* order_ws, void* stream) {
  if (rows <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t* order = order_ws ? support_row_order(ids, width, ld_ids, rows, order_ws, stream) : nullptr;
  const size_t lds = support_lds_bytes(true, H, width);
  support_kernel<true><<<dim3(unsigned(rows)), dim3(NT), lds, s>>>(
      hidden, hidden_dtype, ld_hidden, weight, ld_weight, H, V, temp, temp_scalar, ids, int(width), ld_ids,
      targets, fallback, logprob, entropy, status, fb_list, fb_count, order);
  return int(hipGetLastError());
}

}  // namespace vs

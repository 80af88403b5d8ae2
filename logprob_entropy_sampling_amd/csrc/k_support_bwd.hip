// Backward of recorded-support scoring through the fused projection (SkyRL
// PR #2004, Implementation: gradients through the replayed support's
// logprob and entropy; the description: a singleton support has exactly zero
// entropy and zero entropy gradient).
//
// Over the support S_t of row t the scores are those of p = softmax(z_S), so
//   dX[t, j]    = (a_t ([id_j = y_t] - p_j) - b_t p_j (ln p_j + H_S)) / tau_t
//   d_hidden[t] = sum_j dX[t, j] W[id_j]                         (j ascending)
//   d_weight[v] = sum over pairs (t, j) with id_j = v of dX[t, j] bf16(hidden[t])
//                                                               ((t, j) ascending)
// with the logprob term dropped when y_t is not in S_t (its logprob is the
// constant -inf) and no gradient at all for bad or empty rows.
//
// Kernels:
//   support_grad_kernel  one workgroup per row: the forward's id checks, the
//                        hidden row in LDS, one wave per id for the support
//                        logits, wave 0's fold, dX per id (LDS and a [T][width]
//                        workspace array), then d_hidden by 8-wide chunks of H
//                        over the ids in order; each id of a scored row is
//                        counted into cnt[id].
//   span_sum_kernel, scan_one_kernel, span_scan_kernel
//                        exclusive scan of cnt into offs (the totals of spans of
//                        8192 ids, their scan, then each span from its offset);
//                        fill = 0.
//   pair_scatter_kernel  every counted pair into its id's bucket (any order).
//   weight_grad_kernel   one workgroup per vocabulary row: its bucket sorted by
//                        pair index (so the sum's order is fixed), then
//                        d_weight[v] by 8-wide chunks of H; rows without pairs
//                        are written as zeros.
#include "common.h"
#include "launch.h"

namespace vs {

namespace {

constexpr int NT = 256;
constexpr int kScanThreads = 1024;
constexpr int kSortMax = 4096;  // bucket entries sorted in LDS; longer buckets take ordered block minima

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(uint4 w, uint4 h, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, h.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, h.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, h.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, h.w), acc, false);
  return acc;
}

// acc[0..7] += s * (8 bf16 values of v)
__device__ __forceinline__ void axpy8(float s, uint4 v, float (&acc)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] = __builtin_fmaf(s, bf16_lo(w[e]), acc[2 * e]);
    acc[2 * e + 1] = __builtin_fmaf(s, bf16_hi(w[e]), acc[2 * e + 1]);
  }
}

__device__ __forceinline__ void store8(float* dst, const float (&acc)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = acc[e];
}

__global__ __launch_bounds__(NT) void support_grad_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight, int64_t ld_w, int64_t H,
    int64_t V, const float* __restrict__ temp, float temp_scalar, const int64_t* __restrict__ ids, int width,
    int64_t ld_ids, const int64_t* __restrict__ targets, const float* __restrict__ grad_logprob,
    const float* __restrict__ grad_entropy, float* __restrict__ d_hidden, int64_t ld_dh, float* __restrict__ dx_out,
    uint8_t* __restrict__ row_ok, int32_t* __restrict__ cnt, const int32_t* __restrict__ order) {
  // no contraction: the fold's arithmetic is the forward's, so a singleton's
  // only term has d = 0 exactly and its gradient is exactly 0
#pragma clang fp contract(off)
  extern __shared__ uint4 dyn[];
  uint4* hs = dyn;
  int64_t* sid = reinterpret_cast<int64_t*>(dyn + H / 8);
  float* sx = reinterpret_cast<float*>(sid + width);  // support logits, then dX
  __shared__ int s_bad, s_count, s_ok;

  const int64_t row = order ? int64_t(order[blockIdx.x]) : int64_t(blockIdx.x);  // (results do not depend on it)
  const int tid = threadIdx.x;
  const int64_t nch = H / 8;
  const float tau = temp ? temp[row] : temp_scalar;
  const int64_t y = targets[row];
  if (tid == 0) {
    s_bad = tau_ok(tau) ? 0 : 1;
    s_count = 0;
    s_ok = 0;
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
  bool ok = s_bad == 0 && s_count > 0 && y >= 0 && y < V;
  if (ok) {
    const uint4* hrow = reinterpret_cast<const uint4*>(hidden + row * ld_h);
    for (int64_t q = tid; q < nch; q += NT) hs[q] = hrow[q];
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
    __syncthreads();
    if (tid < 64) {
      // wave 0: the forward's fold, then dX per id (all 64 lanes active)
      const float c = kLog2e / tau;
      float mx = kNegInf;
      int found = 0;
      for (int j = lane; j < width; j += 64) {
        if (sid[j] < 0) continue;
        mx = fmaxf(mx, sx[j] * c);
        if (sid[j] == y) found = 1;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
      Part p{mx, 0.0f, 0.0f};
      if (mx != kNegInf)
        for (int j = lane; j < width; j += 64) {
          if (sid[j] < 0) continue;
          fold(sx[j] * c - mx, p.s, p.a);
        }
      p = wave_merge_to_lane0(p);
      const float m = __shfl(p.m, 0, 64), s = __shfl(p.s, 0, 64), a = __shfl(p.a, 0, 64);
      const bool hit = __ballot(found) != 0;
      const float l2s = log2_hw(s);
      const float lse2 = m + l2s;
      const bool row_fine = lse2 > -__builtin_inff() && lse2 < __builtin_inff();
      const float h = kLn2 * (l2s - a / s);  // the support entropy (nats)
      const float ga = hit && grad_logprob ? grad_logprob[row] : 0.0f;
      const float gb = grad_entropy ? grad_entropy[row] : 0.0f;
      const float inv_tau = 1.0f / tau;
      for (int j = lane; j < width; j += 64) {
        float dx = 0.0f;
        const int64_t id = sid[j];
        if (row_fine && id >= 0) {
          // log2 p_j, floored so that a zero probability never meets ln p = -inf
          const float l2p = floor_d((sx[j] * c - m) - l2s);
          const float pj = exp2_hw(l2p);
          float dz = -pj * (ga + gb * (kLn2 * l2p + h));
          if (id == y) dz += ga;
          dx = dz * inv_tau;
        }
        sx[j] = dx;
      }
      if (lane == 0) s_ok = row_fine ? 1 : 0;
    }
    __syncthreads();
    ok = s_ok != 0;
  }
  if (tid == 0) row_ok[row] = ok ? 1 : 0;
  for (int j = tid; j < width; j += NT) dx_out[row * int64_t(width) + j] = ok ? sx[j] : 0.0f;
  if (ok && cnt)
    for (int j = tid; j < width; j += NT)
      if (sid[j] >= 0) atomicAdd(&cnt[sid[j]], 1);
  if (!d_hidden) return;
  float* dh = d_hidden + row * ld_dh;
  for (int64_t q = tid; q < nch; q += NT) {
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
      int j = 0;
      // four weight rows' chunks in flight per step, summed in id order
      for (; j + 4 <= width; j += 4) {
        uint4 w[4];
        float g[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t id = sid[j + u];
          g[u] = id >= 0 ? sx[j + u] : 0.0f;
          w[u] = id >= 0 ? stream_load(reinterpret_cast<const uint4*>(weight + id * ld_w) + q) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (sid[j + u] >= 0) axpy8(g[u], w[u], acc);
      }
      for (; j < width; ++j) {
        const int64_t id = sid[j];
        if (id >= 0) axpy8(sx[j], stream_load(reinterpret_cast<const uint4*>(weight + id * ld_w) + q), acc);
      }
    }
    store8(dh + 8 * q, acc);
  }
}

// offs[v] = sum_{u < v} cnt[u], offs[V] = the total; fill[v] = 0.
// Exclusive scan of in[base, base + span) (span = kScanSpan, clipped to n)
// into out, starting from carry; returns the span's total to every thread.
// ITEMS consecutive entries per thread (16-byte loads where aligned), a
// wave scan of the thread totals, then the wave totals in order: integer
// sums, so the result does not depend on the order.
constexpr int kScanItems = 8;
constexpr int64_t kScanSpan = int64_t(kScanThreads) * kScanItems;
__device__ __forceinline__ int32_t scan_span(const int32_t* __restrict__ in, int64_t n, int64_t base, int32_t carry,
                                             int32_t* __restrict__ out, int32_t* wsum) {
  constexpr int NW = kScanThreads / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t k0 = base + int64_t(tid) * kScanItems;
  int32_t v[kScanItems];
  if (k0 + kScanItems <= n) {
    const int4 a = reinterpret_cast<const int4*>(in + k0)[0], b = reinterpret_cast<const int4*>(in + k0)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) v[i] = k0 + i < n ? in[k0 + i] : 0;
  }
  int32_t local = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) local += v[i];
  int32_t incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  __syncthreads();  // wsum is free (an earlier span's readers are done)
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int32_t run = carry + incl - local;
  int32_t total = carry;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) run += wsum[w];
    total += wsum[w];
  }
  if (out) {
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      if (k0 + i < n) out[k0 + i] = run;
      run += v[i];
    }
  }
  return total;
}

// bsum[b] = the total of cnt's span b; fill = 0 over it.
__global__ __launch_bounds__(kScanThreads) void span_sum_kernel(const int32_t* __restrict__ cnt, int64_t V,
                                                                int32_t* __restrict__ bsum, int32_t* __restrict__ fill) {
  __shared__ int32_t wsum[kScanThreads / 64];
  const int64_t base = int64_t(blockIdx.x) * kScanSpan;
  for (int64_t k = base + threadIdx.x; k < V && k < base + kScanSpan; k += kScanThreads) fill[k] = 0;
  const int32_t t = scan_span(cnt, V, base, 0, nullptr, wsum);
  if (threadIdx.x == 0) bsum[blockIdx.x] = t;
}

// One workgroup: exclusive scan of in[0, n) into out[0, n], out[n] the total.
__global__ __launch_bounds__(kScanThreads) void scan_one_kernel(const int32_t* __restrict__ in, int64_t n,
                                                                int32_t* __restrict__ out) {
  __shared__ int32_t wsum[kScanThreads / 64];
  int32_t carry = 0;
  for (int64_t base = 0; base < n; base += kScanSpan) carry = scan_span(in, n, base, carry, out, wsum);
  if (threadIdx.x == 0) out[n] = carry;
}

// offs = exclusive scan of cnt: span b from its offset bpre[b]; offs[V] the total.
__global__ __launch_bounds__(kScanThreads) void span_scan_kernel(const int32_t* __restrict__ cnt, int64_t V,
                                                                 const int32_t* __restrict__ bpre, int64_t nb,
                                                                 int32_t* __restrict__ offs) {
  __shared__ int32_t wsum[kScanThreads / 64];
  scan_span(cnt, V, int64_t(blockIdx.x) * kScanSpan, bpre[blockIdx.x], offs, wsum);
  if (blockIdx.x == 0 && threadIdx.x == 0) offs[V] = bpre[nb];
}

__global__ void pair_scatter_kernel(const int64_t* __restrict__ ids, int width, int64_t ld_ids, int64_t rows,
                                    const uint8_t* __restrict__ row_ok, const int32_t* __restrict__ offs,
                                    int32_t* __restrict__ fill, int32_t* __restrict__ list) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * width) return;
  const int64_t t = i / width, j = i - t * width;
  if (!row_ok[t]) return;
  const int64_t id = ids[t * ld_ids + j];
  if (id < 0) return;
  list[offs[id] + atomicAdd(&fill[id], 1)] = int32_t(i);
}

__global__ __launch_bounds__(NT) void weight_grad_kernel(const uint16_t* __restrict__ hidden, int64_t ld_h, int64_t H,
                                                         int64_t V, int width, const int32_t* __restrict__ offs,
                                                         const int32_t* __restrict__ list,
                                                         const float* __restrict__ dx, float* __restrict__ d_weight,
                                                         int64_t ld_dw) {
  __shared__ int32_t sorted[kSortMax];
  __shared__ int32_t s_next;
  const int tid = threadIdx.x;
  const int64_t nch = H / 8;
  for (int64_t v = blockIdx.x; v < V; v += gridDim.x) {
    const int32_t b0 = offs[v], n = offs[v + 1] - b0;
    float* dw = d_weight + v * ld_dw;
    if (n == 0) {  // zeros, 16 bytes per lane over consecutive addresses
      for (int64_t q = tid; q < 2 * nch; q += NT) {
        float* d = dw + 4 * q;
        d[0] = 0.0f;
        d[1] = 0.0f;
        d[2] = 0.0f;
        d[3] = 0.0f;
      }
      continue;  // uniform across the workgroup
    }
    if (n <= kSortMax) {
      // rank sort: pair indices are distinct, so each one's place is the
      // number of smaller ones in the bucket
      for (int i = tid; i < n; i += NT) {
        const int32_t e = list[b0 + i];
        int r = 0;
        for (int k = 0; k < n; ++k) r += list[b0 + k] < e ? 1 : 0;
        sorted[r] = e;
      }
      __syncthreads();
      for (int64_t q = tid; q < nch; q += NT) {
        float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        for (int k = 0; k < n; ++k) {
          const int32_t e = sorted[k];
          const int64_t t = e / width;
          axpy8(dx[e], reinterpret_cast<const uint4*>(hidden + t * ld_h)[q], acc);
        }
        store8(dw + 8 * q, acc);
      }
      __syncthreads();
    } else {
      // a long bucket: visit its entries in ascending order by block minima
      for (int64_t q0 = 0; q0 < nch; q0 += NT) {
        const int64_t q = q0 + tid;
        float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        int32_t prev = -1;
        for (int k = 0; k < n; ++k) {
          if (tid == 0) s_next = 0x7FFFFFFF;
          __syncthreads();
          int32_t best = 0x7FFFFFFF;
          for (int i = tid; i < n; i += NT) {
            const int32_t e = list[b0 + i];
            if (e > prev && e < best) best = e;
          }
          atomicMin(&s_next, best);
          __syncthreads();
          const int32_t e = s_next;
          __syncthreads();
          prev = e;
          if (q < nch) axpy8(dx[e], reinterpret_cast<const uint4*>(hidden + (e / width) * ld_h)[q], acc);
        }
        if (q < nch) store8(dw + 8 * q, acc);
      }
    }
  }
}

size_t support_bwd_lds(int64_t H, int64_t width) { return size_t(H / 8) * 16 + size_t(width) * 8 + size_t(width) * 4; }

}  // namespace

size_t support_backward_workspace_bytes(int64_t rows, int64_t width, int64_t V) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t nb = size_t((V + kScanSpan - 1) / kScanSpan);
  return up(size_t(rows) * size_t(width) * 4) + up(size_t(rows)) + up(size_t(V) * 4) + up(size_t(V + 1) * 4) +
         up(size_t(V) * 4) + up(size_t(rows) * size_t(width) * 4) + up(nb * 4) + up((nb + 1) * 4) +
         up(size_t(rows) * 8);
}

int launch_support_backward(const uint16_t* hidden, int64_t ld_hidden, const uint16_t* weight, int64_t ld_weight,
                            int64_t rows, int64_t H, int64_t V, const float* temp, float temp_scalar,
                            const int64_t* ids, int64_t width, int64_t ld_ids, const int64_t* targets,
                            const float* grad_logprob, const float* grad_entropy, float* d_hidden, int64_t ld_dh,
                            float* d_weight, int64_t ld_dw, void* workspace, void* stream) {
  if (rows <= 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* p = static_cast<char*>(workspace);
  float* dx = reinterpret_cast<float*>(p);
  p += up(size_t(rows) * size_t(width) * 4);
  uint8_t* row_ok = reinterpret_cast<uint8_t*>(p);
  p += up(size_t(rows));
  int32_t* cnt = reinterpret_cast<int32_t*>(p);
  p += up(size_t(V) * 4);
  int32_t* offs = reinterpret_cast<int32_t*>(p);
  p += up(size_t(V + 1) * 4);
  int32_t* fill = reinterpret_cast<int32_t*>(p);
  p += up(size_t(V) * 4);
  int32_t* list = reinterpret_cast<int32_t*>(p);
  p += up(size_t(rows) * size_t(width) * 4);
  const int64_t nb = (V + kScanSpan - 1) / kScanSpan;
  int32_t* bsum = reinterpret_cast<int32_t*>(p);
  p += up(size_t(nb) * 4);
  int32_t* bpre = reinterpret_cast<int32_t*>(p);
  p += up((nb + 1) * 4);
  int32_t* order_ws = reinterpret_cast<int32_t*>(p);  // the rows' workgroup order, then their id counts
  if (nb > 0x7FFFFFFF) return int(hipErrorInvalidValue);
  if (d_weight) {
    const int rc = launch_zero_i32(cnt, V, stream);
    if (rc) return rc;
  }
  const int32_t* order = support_row_order(ids, width, ld_ids, rows, order_ws, stream);
  support_grad_kernel<<<dim3(unsigned(rows)), dim3(NT), support_bwd_lds(H, width), s>>>(
      hidden, ld_hidden, weight, ld_weight, H, V, temp, temp_scalar, ids, int(width), ld_ids, targets, grad_logprob,
      grad_entropy, d_hidden, ld_dh, dx, row_ok, d_weight ? cnt : nullptr, order);
  int rc = int(hipGetLastError());
  if (rc || !d_weight) return rc;
  span_sum_kernel<<<dim3(unsigned(nb)), dim3(kScanThreads), 0, s>>>(cnt, V, bsum, fill);
  scan_one_kernel<<<dim3(1), dim3(kScanThreads), 0, s>>>(bsum, nb, bpre);
  span_scan_kernel<<<dim3(unsigned(nb)), dim3(kScanThreads), 0, s>>>(cnt, V, bpre, nb, offs);
  const int64_t pairs = rows * width;
  if (pairs > 0) {
    pair_scatter_kernel<<<dim3(unsigned((pairs + 255) / 256)), dim3(256), 0, s>>>(ids, int(width), ld_ids, rows,
                                                                                   row_ok, offs, fill, list);
  }
  int ncu = 0;
  rc = device_cu_count(&ncu);
  if (rc) return rc;
  const int64_t grid = V < int64_t(ncu) * 16 ? V : int64_t(ncu) * 16;
  weight_grad_kernel<<<dim3(unsigned(grid)), dim3(NT), 0, s>>>(hidden, ld_hidden, H, V, int(width), offs, list, dx,
                                                                d_weight, ld_dw);
  return int(hipGetLastError());
}

}  // namespace vs
